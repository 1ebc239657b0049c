// Standalone C++ test of the paged decode library through its C ABI only
// (include/pkd.h), with no Python: reads tests/golden/tiny_decode.txt (the
// tiny workload and the float64 CPU oracle's output), writes the BF16 cache
// with reshape_and_cache_bf16, runs the split-K pass and the combine at
// several split counts and the whole-decode call, and checks every output
// element against the oracle within atol = rtol = 1e-2 and the cache bytes
// against the slot scatter. Exit status 0 when everything matches.
//
//   decode_tiny <path to tiny_decode.txt>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <fstream>
#include <map>
#include <sstream>
#include <string>
#include <vector>

#include "pkd.h"

namespace {

struct Golden {
  uint32_t B = 0, Hq = 0, Hkv = 0, D = 0, bs = 0, max_blocks = 0, pages = 0, T = 0;
  float scale = 0.0f;
  std::vector<int32_t> seq_lens, block_tables, slot_mapping;
  std::vector<uint16_t> q, k, v;
  std::vector<double> out;
};

bool load(const char* path, Golden& g) {
  std::ifstream f(path);
  if (!f) return false;
  std::map<std::string, std::vector<std::string>> fields;
  std::string line;
  while (std::getline(f, line)) {
    if (line.empty() || line[0] == '#') continue;
    std::istringstream is(line);
    std::string name, tok;
    is >> name;
    while (is >> tok) fields[name].push_back(tok);
  }
  const auto& d = fields["dims"];
  if (d.size() != 8) return false;
  uint32_t* dims[8] = {&g.B, &g.Hq, &g.Hkv, &g.D, &g.bs, &g.max_blocks, &g.pages, &g.T};
  for (int i = 0; i < 8; ++i) *dims[i] = uint32_t(std::stoul(d[i]));
  g.scale = std::stof(fields["scale"].at(0));
  for (auto& s : fields["seq_lens"]) g.seq_lens.push_back(std::stoi(s));
  for (auto& s : fields["block_tables"]) g.block_tables.push_back(std::stoi(s));
  for (auto& s : fields["slot_mapping"]) g.slot_mapping.push_back(std::stoi(s));
  for (auto& s : fields["q"]) g.q.push_back(uint16_t(std::stoul(s, nullptr, 16)));
  for (auto& s : fields["k"]) g.k.push_back(uint16_t(std::stoul(s, nullptr, 16)));
  for (auto& s : fields["v"]) g.v.push_back(uint16_t(std::stoul(s, nullptr, 16)));
  for (auto& s : fields["out"]) g.out.push_back(std::stod(s));
  return g.q.size() == size_t(g.B) * g.Hq * g.D && g.k.size() == size_t(g.T) * g.Hkv * g.D &&
         g.v.size() == g.k.size() && g.out.size() == g.q.size() && g.seq_lens.size() == g.B &&
         g.block_tables.size() == size_t(g.B) * g.max_blocks && g.slot_mapping.size() == g.T;
}

double bf16_to_double(uint16_t b) {
  uint32_t u = uint32_t(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

#define HIP_OK(x)                                                              \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));      \
      return 2;                                                                \
    }                                                                          \
  } while (0)

#define PKD_CALL(x)                                                            \
  do {                                                                         \
    int s_ = (x);                                                              \
    if (s_ != PKD_OK) {                                                        \
      std::fprintf(stderr, "%s: %s\n", #x, pkd_status_string(s_));             \
      return 3;                                                                \
    }                                                                          \
  } while (0)

template <typename T>
int upload(T** dev, const std::vector<T>& host) {
  HIP_OK(hipMalloc(reinterpret_cast<void**>(dev), host.size() * sizeof(T)));
  HIP_OK(hipMemcpy(*dev, host.data(), host.size() * sizeof(T), hipMemcpyHostToDevice));
  return 0;
}

// |got - ref| <= 1e-2 + 1e-2 |ref| everywhere; prints the largest error.
bool close(const std::vector<uint16_t>& got, const std::vector<double>& ref, const char* what) {
  double worst = 0.0;
  size_t bad = 0;
  for (size_t i = 0; i < ref.size(); ++i) {
    const double e = std::fabs(bf16_to_double(got[i]) - ref[i]);
    if (!(e <= 1e-2 + 1e-2 * std::fabs(ref[i]))) ++bad;
    if (e > worst || std::isnan(e)) worst = e;
  }
  std::printf("%-34s max |err| %.3e  %s\n", what, worst, bad ? "FAIL" : "ok");
  return bad == 0;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc < 2) {
    std::fprintf(stderr, "usage: %s tiny_decode.txt\n", argv[0]);
    return 1;
  }
  Golden g;
  if (!load(argv[1], g)) {
    std::fprintf(stderr, "cannot read %s\n", argv[1]);
    return 1;
  }
  const size_t pool = size_t(g.pages) * g.bs * g.Hkv * g.D;        // elements per pool
  const std::vector<uint16_t> nan_pool(pool, 0x7FC0);               // never-written rows read as NaN
  uint16_t *q, *k, *v, *kc, *vc, *out;
  int32_t *lens, *bt, *slots;
  if (upload(&q, g.q) || upload(&k, g.k) || upload(&v, g.v) || upload(&kc, nan_pool) ||
      upload(&vc, nan_pool) || upload(&lens, g.seq_lens) || upload(&bt, g.block_tables) ||
      upload(&slots, g.slot_mapping))
    return 2;
  HIP_OK(hipMalloc(reinterpret_cast<void**>(&out), g.out.size() * sizeof(uint16_t)));
  const uint32_t row = g.Hkv * g.D;
  PKD_CALL(reshape_and_cache_bf16(k, v, kc, vc, slots, g.T, g.Hkv, g.D, g.bs, row, row, nullptr));

  // the cache holds each token's rows at its slot, NaN elsewhere
  std::vector<uint16_t> kh(pool), vh(pool), kw(nan_pool), vw(nan_pool);
  HIP_OK(hipMemcpy(kh.data(), kc, pool * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(vh.data(), vc, pool * 2, hipMemcpyDeviceToHost));
  for (uint32_t t = 0; t < g.T; ++t) {
    std::memcpy(&kw[size_t(g.slot_mapping[t]) * row], &g.k[size_t(t) * row], row * 2);
    std::memcpy(&vw[size_t(g.slot_mapping[t]) * row], &g.v[size_t(t) * row], row * 2);
  }
  bool ok = kh == kw && vh == vw;
  std::printf("%-34s %s\n", "reshape_and_cache_bf16 bytes", ok ? "ok" : "FAIL");

  std::vector<uint16_t> got(g.out.size());
  for (uint32_t S : {1u, 3u, 8u}) {
    float* ws;
    HIP_OK(hipMalloc(reinterpret_cast<void**>(&ws),
                     paged_decode_workspace_bytes(g.B, g.Hq, g.D, S)));
    HIP_OK(hipMemset(out, 0xFF, got.size() * 2));
    PKD_CALL(paged_decode_attn_splitk_bf16(q, kc, vc, ws, bt, lens, g.max_blocks, g.Hq, g.Hkv, g.D,
                                         g.bs, g.scale, S, g.Hq * g.D, g.B, 0, nullptr));
    PKD_CALL(paged_decode_attn_reduce(ws, out, lens, g.Hq, g.D, S, g.B, nullptr));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(got.data(), out, got.size() * 2, hipMemcpyDeviceToHost));
    char what[64];
    std::snprintf(what, sizeof what, "split-K + combine, S=%u", S);
    ok = close(got, g.out, what) && ok;
    HIP_OK(hipFree(ws));
  }
  HIP_OK(hipMemset(out, 0xFF, got.size() * 2));
  PKD_CALL(paged_decode_attn_bf16(q, kc, vc, out, bt, lens, g.max_blocks, g.B, g.Hq, g.Hkv, g.D, g.bs,
                                g.scale, g.Hq * g.D, 0, nullptr, 1, nullptr));
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(got.data(), out, got.size() * 2, hipMemcpyDeviceToHost));
  ok = close(got, g.out, "whole decode, num_splits 1") && ok;

  // the decode step with the cache write folded in: a cache holding every
  // token but each sequence's last, then the split-K pass that appends it
  {
    std::vector<int32_t> first_slots(g.slot_mapping);
    std::vector<uint16_t> last_k, last_v;
    uint32_t t0 = 0;
    for (uint32_t b = 0; b < g.B; ++b) {
      const uint32_t L = uint32_t(g.seq_lens[b]);
      const uint32_t last = t0 + L - 1;                // sequences of the fixture are not empty
      first_slots[last] = -1;                           // a negative slot is skipped
      last_k.insert(last_k.end(), &g.k[size_t(last) * row], &g.k[size_t(last + 1) * row]);
      last_v.insert(last_v.end(), &g.v[size_t(last) * row], &g.v[size_t(last + 1) * row]);
      t0 += L;
    }
    uint16_t *kc2, *vc2, *lk, *lv;
    int32_t* slots2;
    if (upload(&kc2, nan_pool) || upload(&vc2, nan_pool) || upload(&slots2, first_slots) ||
        upload(&lk, last_k) || upload(&lv, last_v))
      return 2;
    PKD_CALL(reshape_and_cache_bf16(k, v, kc2, vc2, slots2, g.T, g.Hkv, g.D, g.bs, row, row,
                                    nullptr));
    const uint32_t S = 3;
    float* ws;
    HIP_OK(hipMalloc(reinterpret_cast<void**>(&ws), paged_decode_workspace_bytes(g.B, g.Hq, g.D, S)));
    HIP_OK(hipMemset(out, 0xFF, got.size() * 2));
    PKD_CALL(paged_decode_attn_splitk_append_bf16(q, lk, lv, kc2, vc2, ws, bt, lens, g.max_blocks,
                                                g.Hq, g.Hkv, g.D, g.bs, g.scale, S, g.Hq * g.D, row,
                                                row, g.B, 0, nullptr));
    PKD_CALL(paged_decode_attn_reduce(ws, out, lens, g.Hq, g.D, S, g.B, nullptr));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(got.data(), out, got.size() * 2, hipMemcpyDeviceToHost));
    ok = close(got, g.out, "split-K with append + combine") && ok;
    std::vector<uint16_t> kh2(pool), vh2(pool);
    HIP_OK(hipMemcpy(kh2.data(), kc2, pool * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(vh2.data(), vc2, pool * 2, hipMemcpyDeviceToHost));
    const bool same = kh2 == kw && vh2 == vw;
    std::printf("%-34s %s\n", "appended cache bytes", same ? "ok" : "FAIL");
    ok = ok && same;
    for (void* p2 : {static_cast<void*>(kc2), static_cast<void*>(vc2), static_cast<void*>(lk),
                     static_cast<void*>(lv), static_cast<void*>(slots2), static_cast<void*>(ws)})
      HIP_OK(hipFree(p2));
  }

  // the whole decode on the library's static scratch (no workspace argument)
  HIP_OK(hipMemset(out, 0xFF, got.size() * 2));
  PKD_CALL(paged_decode_attn_bf16_noalloc(q, kc, vc, out, bt, lens, g.max_blocks, g.B, g.Hq, g.Hkv,
                                        g.D, g.bs, g.scale, g.Hq * g.D, 0, 3, nullptr));
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(got.data(), out, got.size() * 2, hipMemcpyDeviceToHost));
  ok = close(got, g.out, "whole decode without workspace") && ok;

  // an invalid call is refused with a status, and nothing runs
  const int st = paged_decode_attn_splitk_bf16(q, kc, vc, nullptr, bt, lens, g.max_blocks, g.Hq,
                                               g.Hkv, g.D, g.bs, g.scale, 2, g.Hq * g.D, g.B, 0,
                                               nullptr);
  std::printf("%-34s %s\n", "null workspace refused", st == PKD_ERR_INVALID_ARG ? "ok" : "FAIL");
  ok = ok && st == PKD_ERR_INVALID_ARG;

  for (void* p : {static_cast<void*>(q), static_cast<void*>(k), static_cast<void*>(v),
                  static_cast<void*>(kc), static_cast<void*>(vc), static_cast<void*>(out),
                  static_cast<void*>(lens), static_cast<void*>(bt), static_cast<void*>(slots)})
    HIP_OK(hipFree(p));
  std::printf("%s\n", ok ? "PASS" : "FAIL");
  return ok ? 0 : 4;
}
