// pkv_abi_client: a plain C++ client of the C ABI, with no Python and no PyTorch.
//
// It owns its device memory (hipMalloc) and its stream (hipStreamCreate), runs one decode step
// through libpagedkv (pkv_kv_append then pkv_paged_decode_attention, and pkv_decode_step on a
// second copy of the pools), and writes the results for a caller to check.
//
//   pkv_abi_client INPUT OUTPUT
//
// INPUT (little-endian): int32 header {batch, num_pages, num_kv_heads, max_blocks, partition_pages},
// then block_tables int32[batch][max_blocks], positions int32[batch], q bf16[batch][4 * num_kv_heads][64],
// k_new, v_new bf16[batch][num_kv_heads][64], k_pool, v_pool bf16[num_pages][num_kv_heads][16][64].
// OUTPUT: k_pool, v_pool after the append, then out f32[batch][4 * num_kv_heads][64] of the two
// calls, then out f32 of pkv_decode_step, then the pools after pkv_decode_step.
// Exit status 0 on success; any library or HIP error is printed and gives status 1.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "pagedkv.h"

namespace {

bool hip_ok(hipError_t e, const char *what) {
  if (e == hipSuccess) return true;
  fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  return false;
}

bool pkv_ok(pkv_status s, const char *what) {
  if (s == PKV_OK) return true;
  fprintf(stderr, "%s: %s\n", what, pkv_status_string(s));
  return false;
}

template <typename T>
bool read_array(FILE *f, std::vector<T> &v, size_t n) {
  v.resize(n);
  return fread(v.data(), sizeof(T), n, f) == n;
}

template <typename T>
bool to_device(const std::vector<T> &h, void **d) {
  if (!hip_ok(hipMalloc(d, h.size() * sizeof(T) + 16), "hipMalloc")) return false;
  return hip_ok(hipMemcpy(*d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice), "hipMemcpy H2D");
}

bool append_to_file(FILE *f, const void *d, size_t bytes) {
  std::vector<unsigned char> h(bytes);
  if (!hip_ok(hipMemcpy(h.data(), d, bytes, hipMemcpyDeviceToHost), "hipMemcpy D2H")) return false;
  return fwrite(h.data(), 1, bytes, f) == bytes;
}

}  // namespace

int main(int argc, char **argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s INPUT OUTPUT\n", argv[0]);
    return 2;
  }
  FILE *in = fopen(argv[1], "rb");
  if (!in) {
    perror("input");
    return 1;
  }
  int32_t hdr[5];
  if (fread(hdr, sizeof(int32_t), 5, in) != 5) {
    fprintf(stderr, "short header\n");
    return 1;
  }
  const int32_t batch = hdr[0], num_pages = hdr[1], hkv = hdr[2], max_blocks = hdr[3], part_pages = hdr[4];
  const int32_t hq = 4 * hkv;
  if (batch <= 0 || num_pages <= 0 || hkv <= 0 || max_blocks <= 0) {
    fprintf(stderr, "bad header\n");
    return 1;
  }
  const size_t pool_elems = (size_t)num_pages * hkv * 16 * 64;
  std::vector<int32_t> bt, pos;
  std::vector<uint16_t> q, kn, vn, kp, vp;
  bool ok = read_array(in, bt, (size_t)batch * max_blocks) && read_array(in, pos, (size_t)batch) &&
            read_array(in, q, (size_t)batch * hq * 64) && read_array(in, kn, (size_t)batch * hkv * 64) &&
            read_array(in, vn, (size_t)batch * hkv * 64) && read_array(in, kp, pool_elems) &&
            read_array(in, vp, pool_elems);
  fclose(in);
  if (!ok) {
    fprintf(stderr, "short input\n");
    return 1;
  }
  std::vector<int32_t> lens(batch);
  for (int32_t b = 0; b < batch; ++b) lens[b] = pos[b] + 1;

  hipStream_t stream;
  if (!hip_ok(hipStreamCreate(&stream), "hipStreamCreate")) return 1;
  void *d_bt, *d_pos, *d_lens, *d_q, *d_kn, *d_vn, *d_kp, *d_vp, *d_kp2, *d_vp2, *d_out, *d_out2, *d_ws = nullptr;
  ok = to_device(bt, &d_bt) && to_device(pos, &d_pos) && to_device(lens, &d_lens) && to_device(q, &d_q) &&
       to_device(kn, &d_kn) && to_device(vn, &d_vn) && to_device(kp, &d_kp) && to_device(vp, &d_vp) &&
       to_device(kp, &d_kp2) && to_device(vp, &d_vp2);
  const size_t out_bytes = (size_t)batch * hq * 64 * sizeof(float);
  ok = ok && hip_ok(hipMalloc(&d_out, out_bytes), "hipMalloc out") && hip_ok(hipMalloc(&d_out2, out_bytes), "hipMalloc out");
  int32_t pp = part_pages;
  if (ok && pp <= 0) pp = pkv_plan_partition_pages(batch, hkv, max_blocks, pkv_device_cu_count());
  const size_t ws_bytes = ok ? pkv_decode_workspace_bytes(batch, hq, max_blocks, pp) : 0;
  // the split workspace starts zeroed once (every call leaves its counters at zero again)
  if (ok && ws_bytes > 0)
    ok = hip_ok(hipMalloc(&d_ws, ws_bytes), "hipMalloc workspace") && hip_ok(hipMemset(d_ws, 0, ws_bytes), "hipMemset");
  if (!ok) return 1;

  // The two calls on the pool copy 1, the fused step on copy 2, all on this program's stream.
  const pkv_pool pool1 = {d_kp, d_vp, num_pages, hkv, 64, 16};
  const pkv_pool pool2 = {d_kp2, d_vp2, num_pages, hkv, 64, 16};
  ok = pkv_ok(pkv_kv_append(&pool1, (const int32_t *)d_bt, max_blocks, (const int32_t *)d_pos, d_kn, d_vn, batch, stream),
              "pkv_kv_append") &&
       pkv_ok(pkv_paged_decode_attention(d_q, d_kp, d_vp, num_pages, (const int32_t *)d_bt, max_blocks,
                                         (const int32_t *)d_lens, d_out, PKV_OUT_F32, batch, hq, hkv, 64, 16, 0.125f, pp,
                                         d_ws, ws_bytes, stream),
              "pkv_paged_decode_attention") &&
       pkv_ok(pkv_decode_step(&pool2, d_q, (const int32_t *)d_bt, max_blocks, (const int32_t *)d_pos, d_kn, d_vn, d_out2,
                              PKV_OUT_F32, batch, hq, 0.125f, pp, d_ws, ws_bytes, stream),
              "pkv_decode_step") &&
       hip_ok(hipStreamSynchronize(stream), "hipStreamSynchronize");
  if (!ok) return 1;

  FILE *out = fopen(argv[2], "wb");
  if (!out) {
    perror("output");
    return 1;
  }
  const size_t pool_bytes = pool_elems * sizeof(uint16_t);
  ok = append_to_file(out, d_kp, pool_bytes) && append_to_file(out, d_vp, pool_bytes) &&
       append_to_file(out, d_out, out_bytes) && append_to_file(out, d_out2, out_bytes) &&
       append_to_file(out, d_kp2, pool_bytes) && append_to_file(out, d_vp2, pool_bytes);
  fclose(out);
  for (void *p : {d_bt, d_pos, d_lens, d_q, d_kn, d_vn, d_kp, d_vp, d_kp2, d_vp2, d_out, d_out2, d_ws})
    if (p) (void)hipFree(p);
  (void)hipStreamDestroy(stream);
  if (!ok) return 1;
  printf("pkv_abi_client ok: batch %d, partition_pages %d\n", batch, pp);
  return 0;
}
