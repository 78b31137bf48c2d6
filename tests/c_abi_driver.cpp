// A caller of the C ABI with no Python and no torch: host code that links
// libchunkattn.so, allocates its own device buffers with the HIP runtime and
// calls the library through include/chunkattn.h only.
//
// It runs dense chunk attention over B=1, H=2, Nq=200, Nkv=500, d=128 (several
// 64-key tiles and ragged tails on both axes), then the same attention split
// into two key ranges (float32 branch outputs) recombined by the LSE merge,
// and writes the outputs as raw little-endian files into the directory given
// as argv[1]:
//   o_dense.bf16 [B,Nq,H,d]  lse_dense.f32 [B,H,Nq]
//   o_merged.bf16 [B,Nq,H,d] lse_merged.f32 [B,H,Nq]
// Inputs are generated here from a counter: element i of tensor s (q: s = 0,
// k: 1, v: 2) is ((hash(i + s * 2^24) >> 13) & 255) - 128, divided by 128,
// with hash(x) = x * 2654435761 mod 2^32; every such value is exact in bf16.
// Exit status 0 on success; a library error prints its status and message.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "chunkattn.h"

namespace {

constexpr int B = 1, H = 2, Nq = 200, Nkv = 500, D = 128, SPLIT = 192;

uint16_t gen_bf16(uint32_t i, uint32_t s) {
  const uint32_t x = (i + s * (1u << 24)) * 2654435761u;
  const float f = (float)((int)((x >> 13) & 255u) - 128) / 128.0f;
  uint32_t bits;
  std::memcpy(&bits, &f, 4);
  return (uint16_t)(bits >> 16);   // exact: the value has at most 8 significant bits
}

bool hip_ok(hipError_t e, const char* what) {
  if (e == hipSuccess) return true;
  std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  return false;
}

bool ca_ok(int st, const char* what) {
  if (st == CA_OK) return true;
  std::fprintf(stderr, "%s: %s (%s)\n", what, ca_status_str(st), ca_last_error());
  return false;
}

template <class T>
bool write_file(const std::string& path, const std::vector<T>& v) {
  FILE* f = std::fopen(path.c_str(), "wb");
  if (!f) return false;
  const size_t n = std::fwrite(v.data(), sizeof(T), v.size(), f);
  std::fclose(f);
  return n == v.size();
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 2) {
    std::fprintf(stderr, "usage: %s OUTPUT_DIR\n", argv[0]);
    return 2;
  }
  const std::string dir = argv[1];
  if (ca_abi_version() != CA_ABI_VERSION) {
    std::fprintf(stderr, "ABI version %d, header %d\n", ca_abi_version(), CA_ABI_VERSION);
    return 1;
  }
  const size_t nq = (size_t)B * Nq * H * D, nkv = (size_t)B * Nkv * H * D, nl = (size_t)B * H * Nq;
  std::vector<uint16_t> hq(nq), hk(nkv), hv(nkv);
  for (size_t i = 0; i < nq; ++i) hq[i] = gen_bf16((uint32_t)i, 0);
  for (size_t i = 0; i < nkv; ++i) hk[i] = gen_bf16((uint32_t)i, 1);
  for (size_t i = 0; i < nkv; ++i) hv[i] = gen_bf16((uint32_t)i, 2);

  void *q, *k, *v, *o, *o1, *o2, *om;
  float *lse, *l1, *l2, *lm;
  if (!hip_ok(hipMalloc(&q, nq * 2), "hipMalloc") || !hip_ok(hipMalloc(&k, nkv * 2), "hipMalloc") ||
      !hip_ok(hipMalloc(&v, nkv * 2), "hipMalloc") || !hip_ok(hipMalloc(&o, nq * 2), "hipMalloc") ||
      !hip_ok(hipMalloc(&o1, nq * 4), "hipMalloc") || !hip_ok(hipMalloc(&o2, nq * 4), "hipMalloc") ||
      !hip_ok(hipMalloc(&om, nq * 2), "hipMalloc") ||
      !hip_ok(hipMalloc((void**)&lse, nl * 4), "hipMalloc") ||
      !hip_ok(hipMalloc((void**)&l1, nl * 4), "hipMalloc") ||
      !hip_ok(hipMalloc((void**)&l2, nl * 4), "hipMalloc") ||
      !hip_ok(hipMalloc((void**)&lm, nl * 4), "hipMalloc"))
    return 1;
  if (!hip_ok(hipMemcpy(q, hq.data(), nq * 2, hipMemcpyHostToDevice), "copy q") ||
      !hip_ok(hipMemcpy(k, hk.data(), nkv * 2, hipMemcpyHostToDevice), "copy k") ||
      !hip_ok(hipMemcpy(v, hv.data(), nkv * 2, hipMemcpyHostToDevice), "copy v"))
    return 1;

  const int64_t qs[3] = {(int64_t)Nq * H * D, H * D, D};
  const int64_t ks[3] = {(int64_t)Nkv * H * D, H * D, D};
  const float scale = 0.08838834764831845f;   // 1 / sqrt(128)
  hipStream_t stream;
  if (!hip_ok(hipStreamCreate(&stream), "hipStreamCreate")) return 1;

  // dense, bf16 output, the library's own schedule choice without a workspace
  if (!ca_ok(ca_chunk_attn_fwd(q, k, v, B, H, Nq, Nkv, D, qs, ks, qs, nullptr, nullptr, 0, 64,
                               Nkv, 64, Nq, scale, nullptr, nullptr, nullptr, o, CA_BF16, lse,
                               CA_SPLIT_NEVER, nullptr, 0, stream),
             "ca_chunk_attn_fwd (dense)"))
    return 1;
  // keys [0, SPLIT) and [SPLIT, Nkv) as two dense calls on offset pointers,
  // float32 outputs, then their LSE merge into bf16
  const uint16_t* k2 = static_cast<const uint16_t*>(k) + (size_t)SPLIT * H * D;
  const uint16_t* v2 = static_cast<const uint16_t*>(v) + (size_t)SPLIT * H * D;
  if (!ca_ok(ca_chunk_attn_fwd(q, k, v, B, H, Nq, SPLIT, D, qs, ks, qs, nullptr, nullptr, 0, 64,
                               SPLIT, 64, Nq, scale, nullptr, nullptr, nullptr, o1, CA_F32, l1,
                               CA_SPLIT_NEVER, nullptr, 0, stream),
             "ca_chunk_attn_fwd (branch 1)") ||
      !ca_ok(ca_chunk_attn_fwd(q, k2, v2, B, H, Nq, Nkv - SPLIT, D, qs, ks, qs, nullptr, nullptr,
                               0, 64, Nkv - SPLIT, 64, Nq, scale, nullptr, nullptr, nullptr, o2,
                               CA_F32, l2, CA_SPLIT_NEVER, nullptr, 0, stream),
             "ca_chunk_attn_fwd (branch 2)") ||
      !ca_ok(ca_lse_merge(o1, l1, o2, l2, CA_F32, om, lm, CA_BF16, B, H, Nq, D, qs, qs, qs, stream),
             "ca_lse_merge"))
    return 1;
  // an argument error is reported synchronously and launches nothing
  if (ca_chunk_attn_fwd(q, k, v, B, H, Nq, Nkv, 96, qs, ks, qs, nullptr, nullptr, 0, 64, Nkv, 64,
                        Nq, scale, nullptr, nullptr, nullptr, o, CA_BF16, lse, CA_SPLIT_NEVER,
                        nullptr, 0, stream) != CA_EUNSUPPORTED) {
    std::fprintf(stderr, "d = 96 was not rejected with CA_EUNSUPPORTED\n");
    return 1;
  }
  if (!hip_ok(hipStreamSynchronize(stream), "hipStreamSynchronize")) return 1;

  std::vector<uint16_t> ho(nq), hom(nq);
  std::vector<float> hl(nl), hlm(nl);
  if (!hip_ok(hipMemcpy(ho.data(), o, nq * 2, hipMemcpyDeviceToHost), "copy o") ||
      !hip_ok(hipMemcpy(hl.data(), lse, nl * 4, hipMemcpyDeviceToHost), "copy lse") ||
      !hip_ok(hipMemcpy(hom.data(), om, nq * 2, hipMemcpyDeviceToHost), "copy o merged") ||
      !hip_ok(hipMemcpy(hlm.data(), lm, nl * 4, hipMemcpyDeviceToHost), "copy lse merged"))
    return 1;
  if (!write_file(dir + "/o_dense.bf16", ho) || !write_file(dir + "/lse_dense.f32", hl) ||
      !write_file(dir + "/o_merged.bf16", hom) || !write_file(dir + "/lse_merged.f32", hlm)) {
    std::fprintf(stderr, "cannot write the outputs into %s\n", dir.c_str());
    return 1;
  }
  for (void* p : {q, k, v, o, o1, o2, om}) (void)hipFree(p);
  for (float* p : {lse, l1, l2, lm}) (void)hipFree(p);
  (void)hipStreamDestroy(stream);
  std::printf("c_abi_driver: dense + split/merge written to %s\n", dir.c_str());
  return 0;
}
