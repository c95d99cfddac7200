/* A C program that drives the attention library through its C ABI only: HIP
 * runtime calls for memory, no PyTorch.  Reads a problem from a directory,
 * runs attn_fwd and attn_bwd on the GPU and writes the outputs back:
 *
 *   abi_gpu_client DIR
 *   DIR/params.txt: B S Hq Hkv Dqk Dv dtype mask window_left window_right
 *                   scale softmax_type dropout_p seed_lo seed_hi offset has_seqlens
 *                   [store_ds]  (1: give attn_bwd attn_bwd_ds_workspace_size
 *                   bytes, the stored-dS backward; default 0)
 *   DIR/{q,k,v,do}.bin  raw tensors of the problem's element type (BSHD)
 *   DIR/alpha.bin       float32 [Hq];  DIR/seqlens.bin int32 [B] if has_seqlens
 *   writes DIR/{o,dq,dk,dv}.bin, DIR/lse.bin (float32 [B,Hq,S]) and, for
 *   sink softmax, DIR/doff.bin (float32 [Hq]).
 * dtype ATTN_FP8 runs attn_fwd_fp8 and attn_bwd_fp8 instead: q, k, v hold
 * E4M3 codes and do E5M2 codes (one byte each), DIR/descales.bin float32 [4]
 * (q, k, v, do) and DIR/ds_scale.bin float32 [1]; O and the gradients are
 * bf16, and DIR/amax.bin (float32 [1]) receives the amax of dS.
 * Exit status 0 on success; any failure prints its cause and exits 1. */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sdpa_attn.h"

static const char* g_dir;

static int fail(const char* what) {
  fprintf(stderr, "abi_gpu_client: %s\n", what);
  return 1;
}

static void* read_file(const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", g_dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  void* buf = malloc(bytes ? bytes : 1);
  const size_t got = fread(buf, 1, bytes, f);
  fclose(f);
  if (got != bytes) {
    free(buf);
    return NULL;
  }
  return buf;
}

static int write_file(const char* name, const void* data, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", g_dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) return 1;
  const size_t put = fwrite(data, 1, bytes, f);
  fclose(f);
  return put != bytes;
}

/* Device copy of a host file of `bytes` bytes. */
static void* upload(const char* name, size_t bytes) {
  void* host = read_file(name, bytes);
  void* dev = NULL;
  if (!host) return NULL;
  if (hipMalloc(&dev, bytes ? bytes : 1) != hipSuccess || hipMemcpy(dev, host, bytes, hipMemcpyHostToDevice) != hipSuccess)
    dev = NULL;
  free(host);
  return dev;
}

static int download(const char* name, const void* dev, size_t bytes) {
  void* host = malloc(bytes ? bytes : 1);
  int rc = hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost) != hipSuccess || write_file(name, host, bytes);
  free(host);
  return rc;
}

int main(int argc, char** argv) {
  if (argc != 2) return fail("usage: abi_gpu_client DIR");
  g_dir = argv[1];
  struct attn_params p;
  memset(&p, 0, sizeof p);
  int has_seqlens = 0, store_ds = 0;
  {
    char path[4096];
    snprintf(path, sizeof path, "%s/params.txt", g_dir);
    FILE* f = fopen(path, "r");
    if (!f) return fail("cannot open params.txt");
    const int n = fscanf(f, "%d %d %d %d %d %d %d %d %d %d %f %d %f %u %u %u %d", &p.batch, &p.seqlen, &p.num_heads,
                         &p.num_gqa_groups, &p.head_dim_qk, &p.head_dim_v, &p.dtype, &p.mask_type, &p.window_left,
                         &p.window_right, &p.scale_factor, &p.softmax_type, &p.dropout_p, &p.dropout_seed_lo,
                         &p.dropout_seed_hi, &p.dropout_offset, &has_seqlens);
    if (n == 17 && fscanf(f, "%d", &store_ds) != 1) store_ds = 0;
    fclose(f);
    if (n != 17) return fail("params.txt needs 17 fields");
  }
  if (attn_validate(&p) != ATTN_OK) return fail("attn_validate rejected the problem");
  const int fp8 = p.dtype == ATTN_FP8;
  const size_t es = fp8 ? 1 : (p.dtype == ATTN_BF16 ? 2 : 4);  /* input element size */
  const size_t eo = fp8 ? 2 : es;                              /* output element size (bf16 for FP8) */
  const size_t rows = (size_t)p.batch * p.seqlen;
  const size_t nq = rows * p.num_heads * p.head_dim_qk, nk = rows * p.num_gqa_groups * p.head_dim_qk;
  const size_t nv = rows * p.num_gqa_groups * p.head_dim_v, no = rows * p.num_heads * p.head_dim_v;
  const size_t nlse = (size_t)p.batch * p.num_heads * p.seqlen;
  const int sink = p.softmax_type != ATTN_SOFTMAX_VANILLA;

  void* q = upload("q.bin", nq * es);
  void* k = upload("k.bin", nk * es);
  void* v = upload("v.bin", nv * es);
  void* d_o = upload("do.bin", no * es);
  float* alpha = (float*)upload("alpha.bin", (size_t)p.num_heads * sizeof(float));
  int32_t* seqlens = has_seqlens ? (int32_t*)upload("seqlens.bin", (size_t)p.batch * sizeof(int32_t)) : NULL;
  if (!q || !k || !v || !d_o || !alpha || (has_seqlens && !seqlens)) return fail("cannot read or upload inputs");

  void *o = NULL, *dq = NULL, *dk = NULL, *dv = NULL, *ws = NULL, *wsf = NULL;
  float *lse = NULL, *doff = NULL, *amax = NULL, *descales = NULL, *ds_scale = NULL;
  const size_t ws_bytes = store_ds ? attn_bwd_ds_workspace_size(&p) : attn_bwd_workspace_size(&p);
  if (store_ds && ws_bytes == 0) return fail("no stored-dS backward for this problem");
  const size_t wsf_bytes = attn_fwd_workspace_size(&p);
  if (hipMalloc(&o, no * eo) != hipSuccess || hipMalloc((void**)&lse, nlse * sizeof(float)) != hipSuccess ||
      hipMalloc(&dq, nq * eo) != hipSuccess || hipMalloc(&dk, nk * eo) != hipSuccess ||
      hipMalloc(&dv, nv * eo) != hipSuccess || hipMalloc((void**)&doff, (size_t)p.num_heads * sizeof(float)) != hipSuccess ||
      hipMalloc(&ws, ws_bytes ? ws_bytes : 1) != hipSuccess || hipMalloc(&wsf, wsf_bytes ? wsf_bytes : 1) != hipSuccess ||
      hipMalloc((void**)&amax, sizeof(float)) != hipSuccess)
    return fail("hipMalloc failed");
  if (fp8) {
    descales = (float*)upload("descales.bin", 4 * sizeof(float));
    ds_scale = (float*)upload("ds_scale.bin", sizeof(float));
    if (!descales || !ds_scale) return fail("cannot read or upload the FP8 scales");
  }

  int rc = fp8 ? attn_fwd_fp8(&p, q, k, v, descales, alpha, seqlens, NULL, o, lse, wsf, wsf_bytes, NULL)
               : attn_fwd(&p, q, k, v, alpha, seqlens, NULL, o, lse, NULL, 0, NULL);
  if (rc != ATTN_OK) return fail(attn_status_string(rc));
  rc = fp8 ? attn_bwd_fp8(&p, q, k, v, o, d_o, lse, descales, ds_scale, amax, alpha, seqlens, NULL, dq, dk, dv,
                          sink ? doff : NULL, ws, ws_bytes, NULL)
           : attn_bwd(&p, q, k, v, o, d_o, lse, alpha, seqlens, NULL, dq, dk, dv, sink ? doff : NULL, ws, ws_bytes,
                      NULL);
  if (rc != ATTN_OK) return fail(attn_status_string(rc));
  if (hipDeviceSynchronize() != hipSuccess) return fail("hipDeviceSynchronize failed");

  if (download("o.bin", o, no * eo) || download("lse.bin", lse, nlse * sizeof(float)) ||
      download("dq.bin", dq, nq * eo) || download("dk.bin", dk, nk * eo) || download("dv.bin", dv, nv * eo) ||
      (sink && download("doff.bin", doff, (size_t)p.num_heads * sizeof(float))) ||
      (fp8 && download("amax.bin", amax, sizeof(float))))
    return fail("cannot write outputs");
  if (fp8) {
    hipFree(descales);
    hipFree(ds_scale);
  }
  hipFree(wsf);
  hipFree(amax);
  hipFree(q);
  hipFree(k);
  hipFree(v);
  hipFree(d_o);
  hipFree(alpha);
  if (seqlens) hipFree(seqlens);
  hipFree(o);
  hipFree(lse);
  hipFree(dq);
  hipFree(dk);
  hipFree(dv);
  hipFree(doff);
  hipFree(ws);
  printf("ok\n");
  return 0;
}
