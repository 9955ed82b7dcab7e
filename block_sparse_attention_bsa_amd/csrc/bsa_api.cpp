// Host side of the C ABI declared in include/bsa.h: argument validation, partition and plan
// construction, workspace layouts, and dispatch to the HIP kernel launchers.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <utility>

#include "bsa_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return BSA_OK;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int check_partition(const bsa_partition* part, const char* name) {
  if (part->kind == BSA_PART_FLAT) {
    if (part->flat < 1) return fail(BSA_EINVAL, "%s: flat block size must be >= 1", name);
  } else if (part->kind == BSA_PART_TILE) {
    if (part->bt < 1 || part->bh < 1 || part->bw < 1)
      return fail(BSA_EINVAL, "%s: tile extents must be >= 1", name);
  } else {
    return fail(BSA_EINVAL, "%s: unknown partition kind %d", name, part->kind);
  }
  return BSA_OK;
}

int64_t partition_count(int T, int Hg, int Wg, const bsa_partition* part) {
  const int64_t N = (int64_t)T * Hg * Wg;
  if (part->kind == BSA_PART_FLAT) return ceil_div(N, part->flat);
  return ceil_div(T, part->bt) * ceil_div(Hg, part->bh) * ceil_div(Wg, part->bw);
}

// Fill perm / blk_start for a validated partition; blk_start has nblk + 1 entries.
void partition_fill(int T, int Hg, int Wg, const bsa_partition* part, int32_t* perm,
                    int32_t* blk_start) {
  const int64_t N = (int64_t)T * Hg * Wg;
  if (part->kind == BSA_PART_FLAT) {
    const int64_t nb = ceil_div(N, part->flat);
    for (int64_t n = 0; n < N; ++n) perm[n] = (int32_t)n;
    for (int64_t j = 0; j <= nb; ++j) blk_start[j] = (int32_t)std::min<int64_t>(j * part->flat, N);
    return;
  }
  const int nbt = (int)ceil_div(T, part->bt), nbh = (int)ceil_div(Hg, part->bh),
            nbw = (int)ceil_div(Wg, part->bw);
  int64_t pos = 0, j = 0;
  for (int a = 0; a < nbt; ++a)
    for (int b = 0; b < nbh; ++b)
      for (int c = 0; c < nbw; ++c, ++j) {
        blk_start[j] = (int32_t)pos;
        const int t1 = std::min(T, (a + 1) * part->bt), h1 = std::min(Hg, (b + 1) * part->bh),
                  w1 = std::min(Wg, (c + 1) * part->bw);
        for (int t = a * part->bt; t < t1; ++t)
          for (int h = b * part->bh; h < h1; ++h)
            for (int w = c * part->bw; w < w1; ++w) perm[pos++] = (t * Hg + h) * Wg + w;
      }
  blk_start[j] = (int32_t)pos;
}

int check_device(const bsa_plan* p) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess)
    return fail(BSA_EHIP, "hipGetDevice failed: no usable HIP device");
  if (dev != p->device)
    return fail(BSA_EINVAL, "current device %d differs from the plan's device %d", dev,
                p->device);
  return BSA_OK;
}

int launch_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(BSA_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool supported_attention(const bsa_problem& pr) {
  return (pr.d == 64 || pr.d == 128) && (pr.dtype == BSA_BF16 || pr.dtype == BSA_FP32);
}

template <typename T>
int upload(const std::vector<T>& h, T** d) {
  if (hipMalloc((void**)d, std::max<size_t>(1, h.size()) * sizeof(T)) != hipSuccess) return -1;
  if (!h.empty() &&
      hipMemcpy(*d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice) != hipSuccess)
    return -1;
  return 0;
}

void free_plan(bsa_plan* p) {
  if (!p) return;
  for (void* ptr : {(void*)p->qperm, (void*)p->qstart, (void*)p->kvperm, (void*)p->kvstart,
                    (void*)p->items, (void*)p->fitems, (void*)p->qitem0, (void*)p->kvitems,
                    (void*)p->scale,
                    (void*)p->local_ptr, (void*)p->local_idx, (void*)p->kv_of})
    if (ptr) (void)hipFree(ptr);
  delete p;
}

}  // namespace

SelectWs select_ws_layout(const bsa_plan& p) {
  SelectWs w;
  const size_t rows = (size_t)p.prob.B * p.prob.H * p.nq;
  w.nwords = (p.nkv + 31) / 32;
  w.bitmap = 0;
  w.base_counts = align_up(rows * w.nwords * 4);
  w.head_k = w.base_counts + align_up(rows * 4);
  const size_t BH = (size_t)p.prob.B * p.prob.H;
  w.partial = w.head_k + align_up(BH * 4);
  w.core = w.partial + align_up((rows + 1023) / 1024 * 4);
  w.eg_nrchunk = (int)(((size_t)p.prob.H * p.nq + kEgRowChunk - 1) / kEgRowChunk);
  w.eg_rowent = w.core;
  w.eg_route = w.eg_rowent + align_up(rows * 8);
  w.eg_members = w.eg_route + align_up(BH * 4);
  w.eg_groups = w.eg_members + align_up(BH * 4);
  w.eg_hist = w.eg_groups + align_up(BH * kEgGroupBytes);
  w.eg_bnd = w.eg_hist + align_up(BH * kEgHistBytes);
  w.total = w.eg_bnd + align_up(BH * (size_t)w.eg_nrchunk * 4);
  return w;
}

TokWs tok_ws_layout(const bsa_plan& p) {
  TokWs w;
  const size_t rows = (size_t)p.prob.B * p.prob.H * p.nq;
  w.nwords = (p.nkv + 31) / 32;
  const size_t kb = (size_t)p.prob.B * p.prob.H * p.nkv * 128 * 2;
  w.khi = 0;
  w.klo = align_up(kb);
  w.bitmap = w.klo + align_up(kb);
  w.counts = w.bitmap + align_up(rows * w.nwords * 4);
  w.partial = w.counts + align_up(rows * 4);
  w.total = w.partial + align_up((rows + 1023) / 1024 * 4);
  return w;
}

BwdWs bwd_ws_layout(const bsa_plan& p) {
  BwdWs w;
  const size_t BH = (size_t)p.prob.B * p.prob.H;
  const size_t cols = BH * p.nkv, rows = BH * p.nq;
  w.nwords = (p.nkv + 31) / 32;
  w.delta = 0;
  w.bitmap = align_up(BH * p.prob.N * 4);
  w.col_cnt = w.bitmap + align_up(rows * w.nwords * 4);
  w.col_ptr = w.col_cnt + align_up(cols * 4);
  w.row_idx = w.col_ptr + align_up((cols + 1) * 4);
  const size_t perm_bytes = BH * (size_t)(p.prob.N + kPermPad) * p.prob.d * 2;
  w.kp = w.row_idx + align_up(rows * p.nkv * 4);
  w.vp = w.kp + align_up(perm_bytes);
  w.qp = w.vp + align_up(perm_bytes);
  w.gp = w.qp + align_up(perm_bytes);
  w.lsep = w.gp + align_up(perm_bytes);
  w.dp = w.lsep + align_up(BH * (size_t)(p.prob.N + kPermPad) * 4);
  w.total = w.dp + align_up(BH * (size_t)(p.prob.N + kPermPad) * 4);
  return w;
}

TgWs tg_ws_layout(const bsa_plan& p) {
  TgWs w;
  const size_t BH = (size_t)p.prob.B * p.prob.H, N = (size_t)p.prob.N;
  const size_t rows = BH * p.nq;
  w.nwords = (p.nkv + 31) / 32;
  w.nchunk = (int)((N + 31) / 32);
  const size_t kb = BH * p.nkv * 128 * 2;
  w.khi = 0;
  w.klo = align_up(kb);
  w.e = w.klo + align_up(kb);
  w.heads = w.e + align_up(BH * N * p.nkv * 4);
  w.hist = w.heads + align_up(BH * kTgHeadBytes);
  w.bnd = w.hist + align_up(BH * ((size_t)kTgBins * 4 + (size_t)kTgBins * 8));
  w.bitmap = w.bnd + align_up(BH * w.nchunk * 4);
  w.counts = w.bitmap + align_up(rows * w.nwords * 4);
  w.partial = w.counts + align_up(rows * 4);
  w.total = w.partial + align_up((rows + 1023) / 1024 * 4);
  return w;
}

FwdWs fwd_ws_layout(const bsa_plan& p) {
  FwdWs w{0, 0, 0};
  if (p.prob.dtype != BSA_BF16 || p.prob.d != 128) return w;  // the VALU paths need none
  const size_t perm_bytes =
      (size_t)p.prob.B * p.prob.H * (size_t)(p.prob.N + kPermPad) * p.prob.d * 2;
  w.kp = 0;
  w.vp = align_up(perm_bytes);
  w.total = w.vp + align_up(perm_bytes);
  return w;
}

CalibWs calib_ws_layout(const bsa_plan& p) {
  CalibWs w;
  const size_t BH = (size_t)p.prob.B * p.prob.H;
  w.lse = 0;
  w.part = align_up(BH * p.prob.N * 4);
  w.kp = w.part + align_up(BH * p.n_items * (size_t)p.nkv * kAttnRows * 4);
  w.vp = w.kp + align_up(BH * (size_t)(p.prob.N + kPermPad) * p.prob.d * 2);
  w.total = w.vp + align_up(BH * (size_t)(p.prob.N + kPermPad) * p.prob.d * 2);
  return w;
}

extern "C" {

const char* bsa_last_error(void) { return g_last_error.c_str(); }

int bsa_partition_build(int32_t T, int32_t Hg, int32_t Wg, const bsa_partition* part,
                        int32_t* perm, int32_t* blk_start, int32_t cap_blocks, int32_t* nblk) {
  if (!part || !perm || !blk_start || !nblk)
    return fail(BSA_EINVAL, "bsa_partition_build: NULL argument");
  if (T < 1 || Hg < 1 || Wg < 1) return fail(BSA_EINVAL, "bsa_partition_build: empty grid");
  if ((int64_t)T * Hg * Wg > INT32_MAX)
    return fail(BSA_EUNSUPPORTED, "bsa_partition_build: grid exceeds 2^31 tokens");
  int rc = check_partition(part, "bsa_partition_build");
  if (rc) return rc;
  const int64_t nb = partition_count(T, Hg, Wg, part);
  *nblk = (int32_t)nb;
  if (nb > cap_blocks)
    return fail(BSA_ECAPACITY, "bsa_partition_build: %lld blocks exceed capacity %d",
                (long long)nb, cap_blocks);
  partition_fill(T, Hg, Wg, part, perm, blk_start);
  return ok();
}

int bsa_plan_create(const bsa_problem* prob, const float* head_scale, bsa_plan** out) {
  if (!prob || !out) return fail(BSA_EINVAL, "bsa_plan_create: NULL argument");
  *out = nullptr;
  const bsa_problem& pr = *prob;
  if (pr.B < 1 || pr.H < 1 || pr.T < 1 || pr.Hg < 1 || pr.Wg < 1 || pr.d < 1)
    return fail(BSA_EINVAL, "bsa_plan_create: B, H, d and the grid must be >= 1");
  if ((int64_t)pr.T * pr.Hg * pr.Wg != (int64_t)pr.N)
    return fail(BSA_EINVAL, "bsa_plan_create: N = %d but T*Hg*Wg = %lld", pr.N,
                (long long)pr.T * pr.Hg * pr.Wg);
  if (pr.dtype != BSA_BF16 && pr.dtype != BSA_FP32)
    return fail(BSA_EINVAL, "bsa_plan_create: unknown dtype %d", pr.dtype);
  if (pr.d != 64 && pr.d != 128)
    return fail(BSA_EUNSUPPORTED, "bsa_plan_create: head dim %d (supported: 64, 128)", pr.d);
  int rc = check_partition(&pr.qpart, "bsa_plan_create qpart");
  if (rc) return rc;
  rc = check_partition(&pr.kvpart, "bsa_plan_create kvpart");
  if (rc) return rc;
  if ((int64_t)pr.B * pr.H > (1 << 24))
    return fail(BSA_EUNSUPPORTED, "bsa_plan_create: B*H too large");
  if (head_scale)
    for (int h = 0; h < pr.H; ++h)
      if (!std::isfinite(head_scale[h]) || !(head_scale[h] > 0.f))
        return fail(BSA_EINVAL, "bsa_plan_create: head_scale[%d] must be finite and > 0", h);

  bsa_plan* p = new bsa_plan();
  p->prob = pr;
  p->nq = (int)partition_count(pr.T, pr.Hg, pr.Wg, &pr.qpart);
  p->nkv = (int)partition_count(pr.T, pr.Hg, pr.Wg, &pr.kvpart);
  p->h_qperm.resize(pr.N);
  p->h_kvperm.resize(pr.N);
  p->h_qstart.resize(p->nq + 1);
  p->h_kvstart.resize(p->nkv + 1);
  partition_fill(pr.T, pr.Hg, pr.Wg, &pr.qpart, p->h_qperm.data(), p->h_qstart.data());
  partition_fill(pr.T, pr.Hg, pr.Wg, &pr.kvpart, p->h_kvperm.data(), p->h_kvstart.data());
  for (int i = 0; i < p->nq; ++i) {
    const int sz = p->h_qstart[i + 1] - p->h_qstart[i];
    p->max_qblk = std::max(p->max_qblk, sz);
    p->h_qitem0.push_back((int32_t)(p->h_items.size() / 2));
    for (int off = 0; off < sz; off += kAttnRows) {
      p->h_items.push_back(i);
      p->h_items.push_back(off);
    }
  }
  p->h_qitem0.push_back((int32_t)(p->h_items.size() / 2));
  for (int j = 0; j < p->nkv; ++j) {
    const int sz = p->h_kvstart[j + 1] - p->h_kvstart[j];
    p->max_kvblk = std::max(p->max_kvblk, sz);
    for (int off = 0; off < sz; off += kAttnRows) {
      p->h_kvitems.push_back(j);
      p->h_kvitems.push_back(off);
    }
  }
  p->n_kvitems = (int)(p->h_kvitems.size() / 2);
  p->n_items = (int)(p->h_items.size() / 2);
  {  // forward work items: the 32-row slots left after 128-row chunks, packed by four, then
     // the 128-row chunks
    std::vector<std::pair<int, int>> slots;
    auto push = [&](const int32_t (&d)[kFItemInts]) {
      p->h_fitems.insert(p->h_fitems.end(), d, d + kFItemInts);
    };
    std::vector<int32_t> full;  // the 128-row chunks' items, placed after the packed ones
    for (int i = 0; i < p->nq; ++i) {
      const int sz = p->h_qstart[i + 1] - p->h_qstart[i];
      int off = 0;
      for (; off + kAttnRows <= sz; off += kAttnRows) {
        int32_t d[kFItemInts] = {1, i, i, i, i};
        for (int w = 0; w < 4; ++w) {
          d[5 + 2 * w] = 0;
          d[6 + 2 * w] = off + 32 * w;
        }
        full.insert(full.end(), d, d + kFItemInts);
      }
      for (; off < sz; off += 32) slots.emplace_back(i, off);
    }
    for (size_t s0 = 0; s0 < slots.size(); s0 += 4) {
      int32_t d[kFItemInts] = {0};
      int nl = 0;
      for (int w = 0; w < 4; ++w) {
        d[5 + 2 * w] = -1;
        d[6 + 2 * w] = 0;
        if (s0 + w >= slots.size()) continue;
        const int i = slots[s0 + w].first;
        int l = 0;
        while (l < nl && d[1 + l] != i) ++l;
        if (l == nl) d[1 + nl++] = i;
        d[5 + 2 * w] = l;
        d[6 + 2 * w] = slots[s0 + w].second;
      }
      d[0] = nl;
      for (int l = nl; l < 4; ++l) d[1 + l] = d[1];
      push(d);
    }
    p->h_fitems.insert(p->h_fitems.end(), full.begin(), full.end());
    p->n_fitems = (int)(p->h_fitems.size() / kFItemInts);
  }
  {  // local kv blocks of every query block, from each token's kv block
    std::vector<int32_t>& kv_of = p->h_kv_of;
    kv_of.assign(pr.N, 0);
    for (int j = 0; j < p->nkv; ++j)
      for (int t = p->h_kvstart[j]; t < p->h_kvstart[j + 1]; ++t) kv_of[p->h_kvperm[t]] = j;
    p->h_local_ptr.assign(1, 0);
    std::vector<int32_t> seen(p->nkv, -1);
    for (int i = 0; i < p->nq; ++i) {
      const size_t first = p->h_local_idx.size();
      for (int t = p->h_qstart[i]; t < p->h_qstart[i + 1]; ++t) {
        const int j = kv_of[p->h_qperm[t]];
        if (seen[j] != i) {
          seen[j] = i;
          p->h_local_idx.push_back(j);
        }
      }
      std::sort(p->h_local_idx.begin() + first, p->h_local_idx.end());
      p->h_local_ptr.push_back((int32_t)p->h_local_idx.size());
    }
  }
  p->h_scale.resize(pr.H);
  for (int h = 0; h < pr.H; ++h)
    p->h_scale[h] = head_scale ? head_scale[h] : (float)(1.0 / std::sqrt((double)pr.d));

  if (hipGetDevice(&p->device) != hipSuccess) {
    free_plan(p);
    return fail(BSA_EHIP, "bsa_plan_create: no usable HIP device");
  }
  // perm arrays carry 32 padding entries (token 0) so that fixed-size scalar reads of a chunk's
  // token ids never leave the allocation.
  std::vector<int32_t> qperm_pad(p->h_qperm), kvperm_pad(p->h_kvperm);
  qperm_pad.resize(qperm_pad.size() + 32, 0);
  kvperm_pad.resize(kvperm_pad.size() + 32, 0);
  if (upload(qperm_pad, &p->qperm) || upload(p->h_qstart, &p->qstart) ||
      upload(kvperm_pad, &p->kvperm) || upload(p->h_kvstart, &p->kvstart) ||
      upload(p->h_items, &p->items) || upload(p->h_qitem0, &p->qitem0) ||
      upload(p->h_fitems, &p->fitems) ||
      upload(p->h_kvitems, &p->kvitems) || upload(p->h_scale, &p->scale) ||
      upload(p->h_local_ptr, &p->local_ptr) || upload(p->h_local_idx, &p->local_idx) ||
      upload(p->h_kv_of, &p->kv_of)) {
    free_plan(p);
    return fail(BSA_EHIP, "bsa_plan_create: device allocation or upload failed");
  }
  *out = p;
  return ok();
}

int bsa_plan_destroy(bsa_plan* plan) {
  if (!plan) return fail(BSA_EINVAL, "bsa_plan_destroy: NULL plan");
  free_plan(plan);
  return ok();
}

int bsa_plan_info(const bsa_plan* plan, int32_t* nq, int32_t* nkv, size_t* ws_select,
                  size_t* ws_calib, size_t* ws_bwd, size_t* ws_fwd) {
  if (!plan) return fail(BSA_EINVAL, "bsa_plan_info: NULL plan");
  if (nq) *nq = plan->nq;
  if (nkv) *nkv = plan->nkv;
  if (ws_select) *ws_select = select_ws_layout(*plan).total;
  if (ws_calib) *ws_calib = calib_ws_layout(*plan).total;
  if (ws_bwd) *ws_bwd = bwd_ws_layout(*plan).total;
  if (ws_fwd) *ws_fwd = fwd_ws_layout(*plan).total;
  return ok();
}

int bsa_plan_blocks(const bsa_plan* plan, int32_t which, int32_t* perm, int32_t* blk_start) {
  if (!plan || !perm || !blk_start) return fail(BSA_EINVAL, "bsa_plan_blocks: NULL argument");
  if (which != 0 && which != 1) return fail(BSA_EINVAL, "bsa_plan_blocks: which must be 0 or 1");
  const auto& pv = which == 0 ? plan->h_qperm : plan->h_kvperm;
  const auto& sv = which == 0 ? plan->h_qstart : plan->h_kvstart;
  std::memcpy(perm, pv.data(), pv.size() * sizeof(int32_t));
  std::memcpy(blk_start, sv.data(), sv.size() * sizeof(int32_t));
  return ok();
}

int bsa_pool(const bsa_plan* plan, int32_t which, const void* X, float* Xbar, void* stream) {
  if (!plan || !X || !Xbar) return fail(BSA_EINVAL, "bsa_pool: NULL argument");
  if (which != 0 && which != 1) return fail(BSA_EINVAL, "bsa_pool: which must be 0 or 1");
  int rc = check_device(plan);
  if (rc) return rc;
  return launch_status(launch_pool(*plan, which, X, Xbar, (hipStream_t)stream), "bsa_pool");
}

int bsa_pool_qk(const bsa_plan* plan, const void* Q, const void* K, float* Qbar, float* Kbar,
                void* stream) {
  if (!plan || !Q || !K || !Qbar || !Kbar) return fail(BSA_EINVAL, "bsa_pool_qk: NULL argument");
  int rc = check_device(plan);
  if (rc) return rc;
  return launch_status(launch_pool_qk(*plan, Q, Qbar, K, Kbar, (hipStream_t)stream),
                       "bsa_pool_qk");
}

int bsa_score(const bsa_plan* plan, const float* Qbar, const float* Kbar, int32_t norm, float* S,
              void* stream) {
  if (!plan || !Qbar || !Kbar || !S) return fail(BSA_EINVAL, "bsa_score: NULL argument");
  if (norm != BSA_NORM_ROW && norm != BSA_NORM_HEAD)
    return fail(BSA_EINVAL, "bsa_score: norm must be BSA_NORM_ROW or BSA_NORM_HEAD");
  int rc = check_device(plan);
  if (rc) return rc;
  return launch_status(launch_score(*plan, Qbar, Kbar, norm, S, (hipStream_t)stream),
                       "bsa_score");
}

int bsa_calibrate_mass(const bsa_plan* plan, const void* Q, const void* K, float* M, void* ws,
                       size_t ws_bytes, void* stream) {
  if (!plan || !Q || !K || !M) return fail(BSA_EINVAL, "bsa_calibrate_mass: NULL argument");
  if (plan->prob.dtype != BSA_BF16 || plan->prob.d != 128)
    return fail(BSA_EUNSUPPORTED, "bsa_calibrate_mass: bf16 with d = 128 only");
  const size_t need = calib_ws_layout(*plan).total;
  if (!ws || ws_bytes < need)
    return fail(BSA_ECAPACITY, "bsa_calibrate_mass: workspace %zu < %zu bytes", ws_bytes, need);
  int rc = check_device(plan);
  if (rc) return rc;
  return launch_status(
      launch_calibrate(*plan, Q, K, nullptr, M, nullptr, nullptr, ws, (hipStream_t)stream),
      "bsa_calibrate_mass");
}

int bsa_calibrate_mass_fwd(const bsa_plan* plan, const void* Q, const void* K, const void* V,
                           float* M, void* O, float* lse, void* ws, size_t ws_bytes,
                           void* stream) {
  if (!plan || !Q || !K || !V || !M || !O)
    return fail(BSA_EINVAL, "bsa_calibrate_mass_fwd: NULL argument");
  if (plan->prob.dtype != BSA_BF16 || plan->prob.d != 128)
    return fail(BSA_EUNSUPPORTED, "bsa_calibrate_mass_fwd: bf16 with d = 128 only");
  const size_t need = calib_ws_layout(*plan).total;
  if (!ws || ws_bytes < need)
    return fail(BSA_ECAPACITY, "bsa_calibrate_mass_fwd: workspace %zu < %zu bytes", ws_bytes,
                need);
  int rc = check_device(plan);
  if (rc) return rc;
  return launch_status(launch_calibrate(*plan, Q, K, V, M, O, lse, ws, (hipStream_t)stream),
                       "bsa_calibrate_mass_fwd");
}

}  // extern "C"

// Argument checks shared by the selection entry points (`who` names the caller).
static int check_select(const bsa_plan* plan, const float* S, const bsa_select_params* prm,
                        const int32_t* row_ptr, const int32_t* col_idx, int64_t col_cap,
                        const char* who, bool need_S = true) {
  if (!plan || (need_S && !S) || !prm || !row_ptr || !col_idx)
    return fail(BSA_EINVAL, "%s: NULL argument", who);
  if (prm->pool != BSA_POOL_ROW && prm->pool != BSA_POOL_HEAD &&
      prm->pool != BSA_POOL_LOCAL_TOPK)
    return fail(BSA_EINVAL, "%s: unknown pool %d", who, prm->pool);
  if (prm->pool != BSA_POOL_LOCAL_TOPK && !(prm->p > 0.0 && prm->p <= 1.0))
    return fail(BSA_EINVAL, "%s: p must lie in (0, 1]", who);
  if (prm->pool == BSA_POOL_LOCAL_TOPK && (prm->fixed_k < 0 || prm->min_k_mode != BSA_MINK_NONE))
    return fail(BSA_EINVAL, "%s: LOCAL_TOPK takes fixed_k >= 0 and no minimum count", who);
  if (prm->min_k_mode < BSA_MINK_NONE || prm->min_k_mode > BSA_MINK_WEIGHTED_MEAN)
    return fail(BSA_EINVAL, "%s: unknown min_k_mode %d", who, prm->min_k_mode);
  if (prm->min_k_mode == BSA_MINK_FIXED && prm->fixed_k < 0)
    return fail(BSA_EINVAL, "%s: fixed_k must be >= 0", who);
  if (prm->pool == BSA_POOL_LOCAL_TOPK && plan->nkv > 2048)
    return fail(BSA_EUNSUPPORTED, "%s: LOCAL_TOPK supports up to 2048 kv blocks", who);
  if (prm->pool == BSA_POOL_HEAD && prm->min_k_mode != BSA_MINK_NONE)
    return fail(BSA_EUNSUPPORTED, "%s: a minimum count applies to the ROW pool only", who);
  if (plan->nkv > kMaxSelectBlocks)
    return fail(BSA_EUNSUPPORTED, "%s: %d kv blocks exceed the supported %d", who, plan->nkv,
                kMaxSelectBlocks);
  const int64_t need_cols = (int64_t)plan->prob.B * plan->prob.H * plan->nq * plan->nkv;
  if (need_cols > (int64_t)INT32_MAX)  // row_ptr and the scan carries are 32-bit
    return fail(BSA_EUNSUPPORTED, "%s: B * H * nq * nkv exceeds 2^31 - 1", who);
  if (col_cap < need_cols)
    return fail(BSA_ECAPACITY, "%s: col_idx capacity %lld < %lld", who, (long long)col_cap,
                (long long)need_cols);
  return BSA_OK;
}

extern "C" {

int bsa_select(const bsa_plan* plan, const float* S, const bsa_select_params* prm,
               int32_t* row_ptr, int32_t* col_idx, int64_t col_cap, int32_t* counts,
               int32_t* head_k, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_select(plan, S, prm, row_ptr, col_idx, col_cap, "bsa_select");
  if (rc) return rc;
  const size_t need = select_ws_layout(*plan).total;
  if (!ws || ws_bytes < need)
    return fail(BSA_ECAPACITY, "bsa_select: workspace %zu < %zu bytes", ws_bytes, need);
  rc = check_device(plan);
  if (rc) return rc;
  return launch_status(launch_select(*plan, S, *prm, row_ptr, col_idx, counts, head_k, ws,
                                     (hipStream_t)stream),
                       "bsa_select");
}

int bsa_select_noalloc(const bsa_plan* plan, const float* S, const bsa_select_params* prm,
                       int32_t* row_ptr, int32_t* col_idx, int64_t col_cap, int32_t* counts,
                       int32_t* head_k, void* stream) {
  int rc = check_select(plan, S, prm, row_ptr, col_idx, col_cap, "bsa_select_noalloc");
  if (rc) return rc;
  const size_t need = select_ws_layout(*plan).core;
  if (need > kSelectScratchBytes)
    return fail(BSA_ECAPACITY,
                "bsa_select_noalloc: this plan needs %zu bytes of scratch, above the library's "
                "fixed %zu (B * H * nq * ceil(nkv / 32) words); use bsa_select with a workspace",
                need, kSelectScratchBytes);
  rc = check_device(plan);
  if (rc) return rc;
  void* scratch_ptr = nullptr;
  const hipError_t e = select_scratch(&scratch_ptr);
  if (e != hipSuccess)
    return fail(BSA_EHIP, "bsa_select_noalloc: scratch address: %s", hipGetErrorString(e));
  return launch_status(launch_select(*plan, S, *prm, row_ptr, col_idx, counts, head_k,
                                     scratch_ptr, (hipStream_t)stream),
                       "bsa_select_noalloc");
}

int bsa_score_select(const bsa_plan* plan, const float* Qbar, const float* Kbar,
                     const bsa_select_params* prm, float* S, int32_t* row_ptr, int32_t* col_idx,
                     int64_t col_cap, int32_t* counts, int32_t* head_k, void* ws,
                     size_t ws_bytes, void* stream) {
  if (!Qbar || !Kbar) return fail(BSA_EINVAL, "bsa_score_select: NULL argument");
  int rc = check_select(plan, S, prm, row_ptr, col_idx, col_cap, "bsa_score_select", false);
  if (rc) return rc;
  if (prm->pool != BSA_POOL_ROW)
    return fail(BSA_EUNSUPPORTED, "bsa_score_select: the ROW pool only (bsa_score then "
                "bsa_select for the others)");
  if (plan->nkv > kWaveRowMaxBlocks)
    return fail(BSA_EUNSUPPORTED, "bsa_score_select: more than %d kv blocks", kWaveRowMaxBlocks);
  if (prm->min_k_mode != BSA_MINK_NONE && !S)
    return fail(BSA_EINVAL, "bsa_score_select: a minimum count needs S (its top-up reads it)");
  const size_t need = select_ws_layout(*plan).total;
  if (!ws || ws_bytes < need)
    return fail(BSA_ECAPACITY, "bsa_score_select: workspace %zu < %zu bytes", ws_bytes, need);
  rc = check_device(plan);
  if (rc) return rc;
  return launch_status(launch_score_select_csr(*plan, Qbar, Kbar, *prm, S, row_ptr, col_idx,
                                               counts, head_k, ws, (hipStream_t)stream),
                       "bsa_score_select");
}

int bsa_select_eg(const bsa_plan* plan, const float* S, const bsa_eg_params* prm,
                  int32_t* row_ptr, int32_t* col_idx, int64_t col_cap, int32_t* counts,
                  float* head_entropy, int32_t* head_pooled, void* ws, size_t ws_bytes,
                  void* stream) {
  if (!plan || !S || !prm || !row_ptr || !col_idx)
    return fail(BSA_EINVAL, "bsa_select_eg: NULL argument");
  if (!(prm->p > 0.0 && prm->p <= 1.0))
    return fail(BSA_EINVAL, "bsa_select_eg: p must lie in (0, 1]");
  if (std::isnan(prm->theta)) return fail(BSA_EINVAL, "bsa_select_eg: theta is NaN");
  if (prm->group_size < 1)
    return fail(BSA_EINVAL, "bsa_select_eg: group_size must be >= 1");
  if (plan->nkv > kMaxSelectBlocks)
    return fail(BSA_EUNSUPPORTED, "bsa_select_eg: %d kv blocks exceed the supported %d",
                plan->nkv, kMaxSelectBlocks);
  if ((int64_t)plan->prob.H * plan->nq * plan->nkv > (int64_t)INT32_MAX)
    return fail(BSA_EUNSUPPORTED, "bsa_select_eg: H * nq * nkv exceeds 2^31 - 1");
  const int64_t need_cols = (int64_t)plan->prob.B * plan->prob.H * plan->nq * plan->nkv;
  if (col_cap < need_cols)
    return fail(BSA_ECAPACITY, "bsa_select_eg: col_idx capacity %lld < %lld",
                (long long)col_cap, (long long)need_cols);
  const size_t need = select_ws_layout(*plan).total;
  if (!ws || ws_bytes < need)
    return fail(BSA_ECAPACITY, "bsa_select_eg: workspace %zu < %zu bytes", ws_bytes, need);
  int rc = check_device(plan);
  if (rc) return rc;
  return launch_status(launch_select_eg(*plan, S, *prm, row_ptr, col_idx, counts, head_entropy,
                                        head_pooled, ws, (hipStream_t)stream),
                       "bsa_select_eg");
}

int bsa_tokens_ws(const bsa_plan* plan, size_t* ws_bytes) {
  if (!plan || !ws_bytes) return fail(BSA_EINVAL, "bsa_tokens_ws: NULL argument");
  *ws_bytes = tok_ws_layout(*plan).total;
  return BSA_OK;
}

static int check_tokens(const bsa_plan* plan, int32_t k, const char* who) {
  if (plan->prob.dtype != BSA_BF16 || plan->prob.d != 128)
    return fail(BSA_EUNSUPPORTED, "%s: bf16 and d = 128 only", who);
  if (k < 0) return fail(BSA_EINVAL, "%s: k must be >= 0", who);
  if (k > kMaxTokenK) return fail(BSA_EUNSUPPORTED, "%s: k above %d", who, kMaxTokenK);
  if (plan->nkv > 2048)
    return fail(BSA_EUNSUPPORTED, "%s: more than 2048 kv blocks", who);
  return BSA_OK;
}

int bsa_select_tokens(const bsa_plan* plan, const void* Q, const float* Kbar, int32_t k,
                      int32_t* sel, int32_t* row_ptr, int32_t* col_idx, int64_t col_cap,
                      void* ws, size_t ws_bytes, void* stream) {
  if (!plan || !Q || !Kbar || !sel || !row_ptr || !col_idx)
    return fail(BSA_EINVAL, "bsa_select_tokens: NULL argument");
  int rc = check_tokens(plan, k, "bsa_select_tokens");
  if (rc) return rc;
  const int64_t need_cols = (int64_t)plan->prob.B * plan->prob.H * plan->nq * plan->nkv;
  if (need_cols > (int64_t)INT32_MAX)  // row_ptr and the scan carries are 32-bit
    return fail(BSA_EUNSUPPORTED, "bsa_select_tokens: B * H * nq * nkv exceeds 2^31 - 1");
  if (col_cap < need_cols)
    return fail(BSA_ECAPACITY, "bsa_select_tokens: col_idx capacity %lld < %lld",
                (long long)col_cap, (long long)need_cols);
  const size_t need = tok_ws_layout(*plan).total;
  if (!ws || ws_bytes < need)
    return fail(BSA_ECAPACITY, "bsa_select_tokens: workspace %zu < %zu bytes", ws_bytes, need);
  rc = check_device(plan);
  if (rc) return rc;
  return launch_status(launch_select_tokens(*plan, Q, Kbar, k, sel, row_ptr, col_idx, ws,
                                            (hipStream_t)stream),
                       "bsa_select_tokens");
}

int bsa_attn_fwd_tokens(const bsa_plan* plan, const void* Q, const void* K, const void* V,
                        const int32_t* row_ptr, const int32_t* col_idx, const int32_t* sel,
                        int32_t k, void* O, float* lse, void* ws, size_t ws_bytes,
                        void* stream) {
  if (!plan || !Q || !K || !V || !row_ptr || !col_idx || !sel || !O)
    return fail(BSA_EINVAL, "bsa_attn_fwd_tokens: NULL argument");
  int rc = check_tokens(plan, k, "bsa_attn_fwd_tokens");
  if (rc) return rc;
  const size_t need = fwd_ws_layout(*plan).total;
  if (!ws || ws_bytes < need)
    return fail(BSA_ECAPACITY, "bsa_attn_fwd_tokens: workspace %zu < %zu bytes", ws_bytes, need);
  rc = check_device(plan);
  if (rc) return rc;
  const int nslots = 1 + std::min<int>(k, plan->nkv - 1);
  return launch_status(launch_attn_fwd_tokens(*plan, Q, K, V, row_ptr, col_idx, sel, nslots, O,
                                              lse, ws, (hipStream_t)stream),
                       "bsa_attn_fwd_tokens");
}

int bsa_tokens_global_ws(const bsa_plan* plan, size_t* ws_bytes) {
  if (!plan || !ws_bytes) return fail(BSA_EINVAL, "bsa_tokens_global_ws: NULL argument");
  *ws_bytes = tg_ws_layout(*plan).total;
  return BSA_OK;
}

int bsa_select_tokens_global(const bsa_plan* plan, const void* Q, const float* Kbar, double tau,
                             uint32_t* tbits, int32_t* row_ptr, int32_t* col_idx,
                             int64_t col_cap, void* ws, size_t ws_bytes, void* stream) {
  if (!plan || !Q || !Kbar || !tbits || !row_ptr || !col_idx)
    return fail(BSA_EINVAL, "bsa_select_tokens_global: NULL argument");
  if (plan->prob.dtype != BSA_BF16 || plan->prob.d != 128)
    return fail(BSA_EUNSUPPORTED, "bsa_select_tokens_global: bf16 and d = 128 only");
  if (!(tau > 0.0 && tau <= 1.0))
    return fail(BSA_EINVAL, "bsa_select_tokens_global: tau must lie in (0, 1]");
  if (plan->nkv > kWaveRowMaxBlocks)
    return fail(BSA_EUNSUPPORTED, "bsa_select_tokens_global: more than %d kv blocks",
                kWaveRowMaxBlocks);
  const int64_t need_cols = (int64_t)plan->prob.B * plan->prob.H * plan->nq * plan->nkv;
  if (need_cols > (int64_t)INT32_MAX)
    return fail(BSA_EUNSUPPORTED, "bsa_select_tokens_global: B * H * nq * nkv exceeds 2^31 - 1");
  if (col_cap < need_cols)
    return fail(BSA_ECAPACITY, "bsa_select_tokens_global: col_idx capacity %lld < %lld",
                (long long)col_cap, (long long)need_cols);
  const size_t need = tg_ws_layout(*plan).total;
  if (!ws || ws_bytes < need)
    return fail(BSA_ECAPACITY, "bsa_select_tokens_global: workspace %zu < %zu bytes", ws_bytes,
                need);
  int rc = check_device(plan);
  if (rc) return rc;
  return launch_status(launch_select_tokens_global(*plan, Q, Kbar, tau, tbits, row_ptr, col_idx,
                                                   ws, (hipStream_t)stream),
                       "bsa_select_tokens_global");
}

int bsa_attn_fwd_token_bits(const bsa_plan* plan, const void* Q, const void* K, const void* V,
                            const int32_t* row_ptr, const int32_t* col_idx,
                            const uint32_t* tbits, void* O, float* lse, void* ws,
                            size_t ws_bytes, void* stream) {
  if (!plan || !Q || !K || !V || !row_ptr || !col_idx || !tbits || !O)
    return fail(BSA_EINVAL, "bsa_attn_fwd_token_bits: NULL argument");
  if (plan->prob.dtype != BSA_BF16 || plan->prob.d != 128)
    return fail(BSA_EUNSUPPORTED, "bsa_attn_fwd_token_bits: bf16 and d = 128 only");
  if (plan->nkv > kTokBitsMaxBlocks)
    return fail(BSA_EUNSUPPORTED, "bsa_attn_fwd_token_bits: more than %d kv blocks",
                kTokBitsMaxBlocks);
  const size_t need = fwd_ws_layout(*plan).total;
  if (!ws || ws_bytes < need)
    return fail(BSA_ECAPACITY, "bsa_attn_fwd_token_bits: workspace %zu < %zu bytes", ws_bytes,
                need);
  int rc = check_device(plan);
  if (rc) return rc;
  return launch_status(launch_attn_fwd_token_bits(*plan, Q, K, V, row_ptr, col_idx, tbits, O,
                                                  lse, ws, (hipStream_t)stream),
                       "bsa_attn_fwd_token_bits");
}

int bsa_attn_fwd(const bsa_plan* plan, const void* Q, const void* K, const void* V,
                 const int32_t* row_ptr, const int32_t* col_idx, void* O, float* lse, void* ws,
                 size_t ws_bytes, void* stream) {
  if (!plan || !Q || !K || !V || !row_ptr || !col_idx || !O)
    return fail(BSA_EINVAL, "bsa_attn_fwd: NULL argument");
  if (!supported_attention(plan->prob))
    return fail(BSA_EUNSUPPORTED, "bsa_attn_fwd: unsupported dtype/d combination");
  const size_t need = fwd_ws_layout(*plan).total;
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(BSA_ECAPACITY, "bsa_attn_fwd: workspace %zu < %zu bytes", ws_bytes, need);
  int rc = check_device(plan);
  if (rc) return rc;
  return launch_status(launch_attn_fwd(*plan, Q, K, V, row_ptr, col_idx, O, lse, ws,
                                       (hipStream_t)stream),
                       "bsa_attn_fwd");
}

int bsa_attn_bwd(const bsa_plan* plan, const void* Q, const void* K, const void* V,
                 const void* O, const void* dO, const float* lse, const int32_t* row_ptr,
                 const int32_t* col_idx, void* dQ, void* dK, void* dV, void* ws,
                 size_t ws_bytes, void* stream) {
  if (!plan || !Q || !K || !V || !O || !dO || !lse || !row_ptr || !col_idx || !dQ || !dK || !dV)
    return fail(BSA_EINVAL, "bsa_attn_bwd: NULL argument");
  if (plan->prob.dtype != BSA_BF16 || plan->prob.d != 128)
    return fail(BSA_EUNSUPPORTED, "bsa_attn_bwd: bf16 with d = 128 only");
  if ((int64_t)plan->prob.B * plan->prob.H * plan->nq * plan->nkv > (int64_t)INT32_MAX)
    return fail(BSA_EUNSUPPORTED, "bsa_attn_bwd: B * H * nq * nkv exceeds 2^31 - 1 (32-bit CSC)");
  if (plan->nkv > kMaxSelectBlocks)
    return fail(BSA_EUNSUPPORTED, "bsa_attn_bwd: %d kv blocks exceed the supported %d",
                plan->nkv, kMaxSelectBlocks);
  const size_t need = bwd_ws_layout(*plan).total;
  if (!ws || ws_bytes < need)
    return fail(BSA_ECAPACITY, "bsa_attn_bwd: workspace %zu < %zu bytes", ws_bytes, need);
  int rc = check_device(plan);
  if (rc) return rc;
  return launch_status(launch_attn_bwd(*plan, Q, K, V, O, dO, lse, row_ptr, col_idx, dQ, dK, dV,
                                       ws, (hipStream_t)stream),
                       "bsa_attn_bwd");
}

}  // extern "C"
