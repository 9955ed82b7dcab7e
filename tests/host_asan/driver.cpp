// Exercises the library's host code through the C ABI in a CPU-only build (host_stubs.cpp stands
// in for the device): plans for every workload shape and kv partition, partition copies into
// buffers of exactly the documented size, every entry point with valid arguments, and the error
// paths. Run under AddressSanitizer and UndefinedBehaviorSanitizer; exits non-zero on a failed
// check (the sanitizers abort on their own findings).
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "bsa.h"

extern int g_launches;

static int g_fail = 0;
#define CHECK(c)                                                                 \
  do {                                                                           \
    if (!(c)) {                                                                  \
      std::fprintf(stderr, "check failed at line %d: %s (%s)\n", __LINE__, #c,    \
                   bsa_last_error());                                            \
      ++g_fail;                                                                  \
    }                                                                            \
  } while (0)

static bsa_partition tile(int bt, int bh, int bw) { return bsa_partition{BSA_PART_TILE, 0, bt, bh, bw}; }
static bsa_partition flat(int s) { return bsa_partition{BSA_PART_FLAT, s, 0, 0, 0}; }

// A device-pointer stand-in: the stub launchers never dereference it, so one small buffer
// serves every argument; only the sizes passed alongside are checked by the library.
alignas(256) static char g_dev[256];
struct Buf {
  explicit Buf(size_t) {}
  void* p() { return g_dev; }
  float* f() { return reinterpret_cast<float*>(g_dev); }
  int32_t* i() { return reinterpret_cast<int32_t*>(g_dev); }
};

static void exercise(int B, int H, int d, int dtype, int T, int Hg, int Wg, bsa_partition qp,
                     bsa_partition kp) {
  const int N = T * Hg * Wg;
  bsa_problem pr{B, H, N, d, dtype, T, Hg, Wg, qp, kp};
  std::vector<float> hs(H);
  for (int h = 0; h < H; ++h) hs[h] = 0.05f + 0.01f * h;
  bsa_plan* plan = nullptr;
  CHECK(bsa_plan_create(&pr, hs.data(), &plan) == BSA_OK);
  if (!plan) return;
  int32_t nq = 0, nkv = 0;
  size_t wss = 0, wsc = 0, wsb = 0, wsf = 0;
  CHECK(bsa_plan_info(plan, &nq, &nkv, &wss, &wsc, &wsb, &wsf) == BSA_OK);
  CHECK(bsa_plan_info(plan, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == BSA_OK);
  for (int which = 0; which < 2; ++which) {
    const int nb = which ? nkv : nq;
    std::vector<int32_t> perm(N), start(nb + 1);  // exactly the documented sizes
    CHECK(bsa_plan_blocks(plan, which, perm.data(), start.data()) == BSA_OK);
    std::vector<char> seen(N, 0);
    for (int n : perm) {
      CHECK(n >= 0 && n < N);
      if (n >= 0 && n < N) seen[n]++;
    }
    for (int n = 0; n < N; ++n) CHECK(seen[n] == 1);
    CHECK(start[0] == 0 && start[nb] == N);
    // the same partition from the host-only builder
    std::vector<int32_t> perm2(N), start2(nb + 1);
    int32_t nb2 = 0;
    CHECK(bsa_partition_build(T, Hg, Wg, which ? &kp : &qp, perm2.data(), start2.data(), nb,
                              &nb2) == BSA_OK);
    CHECK(nb2 == nb && perm2 == perm && start2 == start);
    if (nb > 1) {  // one block short: capacity error, nothing written past the buffer
      std::vector<int32_t> small(nb);
      CHECK(bsa_partition_build(T, Hg, Wg, which ? &kp : &qp, perm2.data(), small.data(),
                                nb - 1, &nb2) == BSA_ECAPACITY);
      CHECK(nb2 == nb);
    }
  }
  const size_t esz = dtype == BSA_BF16 ? 2 : 4;
  const size_t act = (size_t)B * H * N * d * esz;
  const size_t rows = (size_t)B * H * nq;
  Buf q(act), k(act), v(act), o(act), dout(act), dq(act), dk(act), dv(act);
  Buf qbar((size_t)B * H * nq * d * 4), kbar((size_t)B * H * nkv * d * 4);
  Buf S(rows * nkv * 4), rp((rows + 1) * 4), ci(rows * nkv * 4), cnt(rows * 4), hk(B * H * 4);
  Buf lse((size_t)B * H * N * 4), ws_s(wss), ws_c(wsc), ws_b(wsb), ws_f(wsf);
  const int64_t cap = (int64_t)rows * nkv;
  const int before = g_launches;
  CHECK(bsa_pool(plan, 0, q.p(), qbar.f(), nullptr) == BSA_OK);
  CHECK(bsa_pool_qk(plan, q.p(), k.p(), qbar.f(), kbar.f(), nullptr) == BSA_OK);
  CHECK(bsa_score(plan, qbar.f(), kbar.f(), BSA_NORM_ROW,
                  (float*)S.p(), nullptr) == BSA_OK);
  const bsa_select_params prm[] = {{0.9, BSA_POOL_ROW, BSA_MINK_NONE, 0},
                                   {0.9, BSA_POOL_ROW, BSA_MINK_WEIGHTED_MEAN, 0},
                                   {0.9, BSA_POOL_ROW, BSA_MINK_FIXED, 5},
                                   {0.25, BSA_POOL_HEAD, BSA_MINK_NONE, 0},
                                   {1.0, BSA_POOL_LOCAL_TOPK, BSA_MINK_NONE, 6}};
  for (const auto& pm : prm) {
    const int rc = bsa_select(plan, (float*)S.p(), &pm, (int32_t*)rp.p(), (int32_t*)ci.p(), cap,
                              (int32_t*)cnt.p(), (int32_t*)hk.p(), ws_s.p(), wss, nullptr);
    CHECK(rc == BSA_OK || (pm.pool == BSA_POOL_LOCAL_TOPK && nkv > 2048));
    // workspace one byte short, capacity one short
    CHECK(bsa_select(plan, (float*)S.p(), &pm, (int32_t*)rp.p(), (int32_t*)ci.p(), cap, nullptr,
                     nullptr, ws_s.p(), wss - 1, nullptr) != BSA_OK);
    CHECK(bsa_select(plan, (float*)S.p(), &pm, (int32_t*)rp.p(), (int32_t*)ci.p(), cap - 1,
                     nullptr, nullptr, ws_s.p(), wss, nullptr) != BSA_OK);
  }
  const bsa_select_params badp[] = {{0.0, BSA_POOL_ROW, BSA_MINK_NONE, 0},
                                    {1.5, BSA_POOL_ROW, BSA_MINK_NONE, 0},
                                    {0.9, 7, BSA_MINK_NONE, 0},
                                    {0.9, BSA_POOL_ROW, 9, 0},
                                    {0.9, BSA_POOL_ROW, BSA_MINK_FIXED, -1},
                                    {0.9, BSA_POOL_LOCAL_TOPK, BSA_MINK_FIXED, 2}};
  for (const auto& pm : badp)
    CHECK(bsa_select(plan, (float*)S.p(), &pm, (int32_t*)rp.p(), (int32_t*)ci.p(), cap, nullptr,
                     nullptr, ws_s.p(), wss, nullptr) == BSA_EINVAL);
  const bsa_select_params head_mink{0.9, BSA_POOL_HEAD, BSA_MINK_WEIGHTED_MEAN, 0};
  CHECK(bsa_select(plan, (float*)S.p(), &head_mink, (int32_t*)rp.p(), (int32_t*)ci.p(), cap,
                   nullptr, nullptr, ws_s.p(), wss, nullptr) == BSA_EUNSUPPORTED);
  for (const auto& pm : prm) {  // the allocation-free variant: same checks, no workspace
    const int rc = bsa_select_noalloc(plan, (float*)S.p(), &pm, (int32_t*)rp.p(),
                                      (int32_t*)ci.p(), cap, nullptr, nullptr, nullptr);
    const bool fits = (size_t)rows * ((nkv + 31) / 32) * 4 + rows * 4 + B * H * 4 + 1024 <=
                      (size_t(8) << 20);
    if (pm.pool == BSA_POOL_LOCAL_TOPK && nkv > 2048)
      CHECK(rc == BSA_EUNSUPPORTED);
    else if (fits)
      CHECK(rc == BSA_OK);
    CHECK(bsa_select_noalloc(plan, (float*)S.p(), &pm, (int32_t*)rp.p(), (int32_t*)ci.p(),
                             cap - 1, nullptr, nullptr, nullptr) != BSA_OK);
  }
  for (const auto& pm : prm) {  // the fused score-and-select: ROW pool only
    const int rc = bsa_score_select(plan, qbar.f(), kbar.f(), &pm, S.f(), rp.i(), ci.i(), cap,
                                    cnt.i(), hk.i(), ws_s.p(), wss, nullptr);
    if (pm.pool != BSA_POOL_ROW || nkv > 2048)
      CHECK(rc == BSA_EUNSUPPORTED);
    else
      CHECK(rc == BSA_OK);
  }
  {
    const bsa_select_params mk{0.9, BSA_POOL_ROW, BSA_MINK_WEIGHTED_MEAN, 0};
    CHECK(bsa_score_select(plan, qbar.f(), kbar.f(), &mk, nullptr, rp.i(), ci.i(), cap, nullptr,
                           nullptr, ws_s.p(), wss, nullptr) ==
          (nkv > 2048 ? BSA_EUNSUPPORTED : BSA_EINVAL));
    const bsa_select_params p0{0.9, BSA_POOL_ROW, BSA_MINK_NONE, 0};
    CHECK(bsa_score_select(plan, qbar.f(), kbar.f(), &p0, nullptr, rp.i(), ci.i(), cap, nullptr,
                           nullptr, ws_s.p(), wss - 1, nullptr) != BSA_OK);
    CHECK(bsa_score_select(plan, nullptr, kbar.f(), &p0, nullptr, rp.i(), ci.i(), cap, nullptr,
                           nullptr, ws_s.p(), wss, nullptr) == BSA_EINVAL);
  }
  const bsa_eg_params eg{0.9, 0.5, 4};
  CHECK(bsa_select_eg(plan, (float*)S.p(), &eg, (int32_t*)rp.p(), (int32_t*)ci.p(), cap,
                      (int32_t*)cnt.p(), nullptr, nullptr, ws_s.p(), wss, nullptr) == BSA_OK);
  const bsa_eg_params egbad{0.9, 0.5, 0};
  CHECK(bsa_select_eg(plan, (float*)S.p(), &egbad, (int32_t*)rp.p(), (int32_t*)ci.p(), cap,
                      nullptr, nullptr, nullptr, ws_s.p(), wss, nullptr) == BSA_EINVAL);
  const bool mfma = dtype == BSA_BF16 && d == 128;
  CHECK(bsa_attn_fwd(plan, q.p(), k.p(), v.p(), (int32_t*)rp.p(), (int32_t*)ci.p(), o.p(),
                     (float*)lse.p(), ws_f.p(), wsf, nullptr) == BSA_OK);
  if (mfma) {
    CHECK(bsa_attn_fwd(plan, q.p(), k.p(), v.p(), (int32_t*)rp.p(), (int32_t*)ci.p(), o.p(),
                       nullptr, ws_f.p(), wsf - 1, nullptr) == BSA_ECAPACITY);
    CHECK(bsa_calibrate_mass(plan, q.p(), k.p(), (float*)S.p(), ws_c.p(), wsc, nullptr) ==
          BSA_OK);
    CHECK(bsa_calibrate_mass(plan, q.p(), k.p(), (float*)S.p(), ws_c.p(), wsc - 1, nullptr) ==
          BSA_ECAPACITY);
    CHECK(bsa_calibrate_mass_fwd(plan, q.p(), k.p(), v.p(), (float*)S.p(), o.p(),
                                 (float*)lse.p(), ws_c.p(), wsc, nullptr) == BSA_OK);
    CHECK(bsa_attn_bwd(plan, q.p(), k.p(), v.p(), o.p(), dout.p(), (float*)lse.p(),
                       (int32_t*)rp.p(), (int32_t*)ci.p(), dq.p(), dk.p(), dv.p(), ws_b.p(), wsb,
                       nullptr) == BSA_OK);
    CHECK(bsa_attn_bwd(plan, q.p(), k.p(), v.p(), o.p(), dout.p(), (float*)lse.p(),
                       (int32_t*)rp.p(), (int32_t*)ci.p(), dq.p(), dk.p(), dv.p(), ws_b.p(),
                       wsb - 1, nullptr) == BSA_ECAPACITY);
    size_t wst = 0;
    CHECK(bsa_tokens_ws(plan, &wst) == BSA_OK);
    Buf ws_t(wst), sel((size_t)B * H * N * 25 * 4);
    const int rc = bsa_select_tokens(plan, q.p(), (float*)kbar.p(), 6, (int32_t*)sel.p(),
                                     (int32_t*)rp.p(), (int32_t*)ci.p(), cap, ws_t.p(), wst,
                                     nullptr);
    CHECK(rc == (nkv > 2048 ? BSA_EUNSUPPORTED : BSA_OK));
    CHECK(bsa_select_tokens(plan, q.p(), (float*)kbar.p(), 25, (int32_t*)sel.p(),
                            (int32_t*)rp.p(), (int32_t*)ci.p(), cap, ws_t.p(), wst,
                            nullptr) == BSA_EUNSUPPORTED);
    size_t wsg = 0;
    CHECK(bsa_tokens_global_ws(plan, &wsg) == BSA_OK);
    Buf ws_g(wsg);
    CHECK(bsa_select_tokens_global(plan, q.p(), kbar.f(), 0.25, (uint32_t*)sel.p(), rp.i(),
                                   ci.i(), cap, ws_g.p(), wsg, nullptr) ==
          (nkv > 2048 ? BSA_EUNSUPPORTED : BSA_OK));
    CHECK(bsa_select_tokens_global(plan, q.p(), kbar.f(), 0.0, (uint32_t*)sel.p(), rp.i(),
                                   ci.i(), cap, ws_g.p(), wsg, nullptr) == BSA_EINVAL);
    CHECK(bsa_select_tokens_global(plan, q.p(), kbar.f(), 0.25, (uint32_t*)sel.p(), rp.i(),
                                   ci.i(), cap, ws_g.p(), wsg - 1, nullptr) != BSA_OK);
    CHECK(bsa_attn_fwd_token_bits(plan, q.p(), k.p(), v.p(), rp.i(), ci.i(), (uint32_t*)sel.p(),
                                  o.p(), nullptr, ws_f.p(), wsf, nullptr) ==
          (nkv > 2048 ? BSA_EUNSUPPORTED : BSA_OK));
    if (nkv <= 2048) {
      CHECK(bsa_attn_fwd_tokens(plan, q.p(), k.p(), v.p(), (int32_t*)rp.p(), (int32_t*)ci.p(),
                                (int32_t*)sel.p(), 6, o.p(), nullptr, ws_f.p(), wsf,
                                nullptr) == BSA_OK);
      CHECK(bsa_attn_fwd_tokens(plan, q.p(), k.p(), v.p(), (int32_t*)rp.p(), (int32_t*)ci.p(),
                                (int32_t*)sel.p(), 6, o.p(), nullptr, ws_f.p(), wsf - 1,
                                nullptr) == BSA_ECAPACITY);
    }
  } else {
    CHECK(bsa_calibrate_mass(plan, q.p(), k.p(), (float*)S.p(), ws_c.p(), wsc, nullptr) ==
          BSA_EUNSUPPORTED);
    CHECK(bsa_attn_bwd(plan, q.p(), k.p(), v.p(), o.p(), dout.p(), (float*)lse.p(),
                       (int32_t*)rp.p(), (int32_t*)ci.p(), dq.p(), dk.p(), dv.p(), ws_b.p(), wsb,
                       nullptr) == BSA_EUNSUPPORTED);
  }
  CHECK(bsa_score(plan, (float*)qbar.p(), (float*)kbar.p(), 5, (float*)S.p(), nullptr) ==
        BSA_EINVAL);
  CHECK(bsa_pool(plan, 2, q.p(), qbar.f(), nullptr) == BSA_EINVAL);
  CHECK(g_launches > before);
  CHECK(bsa_plan_destroy(plan) == BSA_OK);
}

int main() {
  // the five workload shapes (the training workload with each of its kv partitions)
  exercise(1, 2, 64, BSA_FP32, 4, 8, 8, flat(32), flat(32));
  exercise(1, 12, 128, BSA_BF16, 21, 30, 52, tile(4, 4, 8), tile(4, 4, 8));
  exercise(1, 24, 128, BSA_BF16, 33, 45, 80, tile(4, 4, 8), tile(4, 4, 8));
  exercise(1, 40, 128, BSA_BF16, 21, 45, 80, tile(4, 4, 8), tile(3, 45, 80));
  exercise(1, 40, 128, BSA_BF16, 21, 45, 80, tile(4, 4, 8), tile(21, 15, 5));
  exercise(1, 40, 128, BSA_BF16, 21, 45, 80, tile(4, 4, 8), tile(7, 9, 20));
  // ragged edges, batches, flat partitions that do not divide N, one-token blocks, tiles larger
  // than the grid
  exercise(2, 3, 128, BSA_BF16, 5, 7, 13, tile(4, 4, 8), tile(2, 3, 5));
  exercise(3, 1, 64, BSA_BF16, 3, 5, 7, flat(10), flat(1));
  exercise(1, 2, 128, BSA_FP32, 2, 3, 3, tile(9, 9, 9), flat(4));
  exercise(1, 1, 128, BSA_BF16, 1, 1, 1, flat(1), flat(1));
  exercise(1, 2, 128, BSA_BF16, 1, 64, 64, flat(1), tile(1, 32, 32));

  // problems rejected at plan creation
  bsa_plan* plan = nullptr;
  bsa_problem bad{1, 2, 255, 64, BSA_FP32, 4, 8, 8, flat(32), flat(32)};
  CHECK(bsa_plan_create(&bad, nullptr, &plan) == BSA_EINVAL && plan == nullptr);
  bsa_problem badd{1, 2, 256, 96, BSA_FP32, 4, 8, 8, flat(32), flat(32)};
  CHECK(bsa_plan_create(&badd, nullptr, &plan) == BSA_EUNSUPPORTED);
  bsa_problem badp{1, 2, 256, 64, BSA_FP32, 4, 8, 8, tile(0, 1, 1), flat(32)};
  CHECK(bsa_plan_create(&badp, nullptr, &plan) == BSA_EINVAL);
  float hs[2] = {1.f, -1.f};
  bsa_problem okp{1, 2, 256, 64, BSA_FP32, 4, 8, 8, flat(32), flat(32)};
  CHECK(bsa_plan_create(&okp, hs, &plan) == BSA_EINVAL);
  // size limits (32-bit CSR offsets), checked before anything is enqueued
  bsa_problem big{1, 64, 8192, 128, BSA_BF16, 8192, 1, 1, flat(1), flat(1)};
  CHECK(bsa_plan_create(&big, nullptr, &plan) == BSA_OK);
  if (plan) {
    char fake[16];
    const bsa_select_params pm{0.9, BSA_POOL_ROW, BSA_MINK_NONE, 0};
    CHECK(bsa_select(plan, (float*)fake, &pm, (int32_t*)fake, (int32_t*)fake, INT64_MAX, nullptr,
                     nullptr, fake, SIZE_MAX, nullptr) == BSA_EUNSUPPORTED);
    CHECK(bsa_select_noalloc(plan, (float*)fake, &pm, (int32_t*)fake, (int32_t*)fake,
                             INT64_MAX, nullptr, nullptr, nullptr) == BSA_EUNSUPPORTED);
    CHECK(bsa_attn_bwd(plan, fake, fake, fake, fake, fake, (float*)fake, (int32_t*)fake,
                       (int32_t*)fake, fake, fake, fake, fake, SIZE_MAX,
                       nullptr) == BSA_EUNSUPPORTED);
    CHECK(bsa_plan_destroy(plan) == BSA_OK);
  }
  // a selection whose workspace exceeds the fixed scratch: 64 heads of the 720p shape
  bsa_problem wide{1, 64, 33 * 45 * 80, 128, BSA_BF16, 33, 45, 80, tile(4, 4, 8), tile(4, 4, 8)};
  CHECK(bsa_plan_create(&wide, nullptr, &plan) == BSA_OK);
  if (plan) {
    char fake[16];
    const bsa_select_params pm{0.9, BSA_POOL_ROW, BSA_MINK_NONE, 0};
    CHECK(bsa_select_noalloc(plan, (float*)fake, &pm, (int32_t*)fake, (int32_t*)fake, INT64_MAX,
                             nullptr, nullptr, nullptr) == BSA_ECAPACITY);
    CHECK(bsa_plan_destroy(plan) == BSA_OK);
  }
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("host checks passed (%d launches recorded)\n", g_launches);
  return 0;
}
