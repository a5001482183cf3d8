// zha_api.hip -- host side of the C ABI declared in include/zha.h: argument
// validation, the tree object and its device workspace, and the launches.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <new>

#include <algorithm>
#include <vector>

#include "zha_internal.h"

int zha_score_wgs(const zha_tree* t, int level);
int zha_compact_chunks(int64_t nodes);
int zha_small_score_rows();
int zha_hist_bins();
int64_t zha_sel_cand_entries(int U);
int zha_sel_ctr_words(int U);
size_t zha_spine_bytes(int L, int d, int R);
size_t zha_build_lds_bytes(int C, int S, int L, int d, int R, int esize);

namespace {

thread_local char g_last_error[256] = "";

zha_status hip_fail(const char* where, hipError_t e) {
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%d)", where, hipGetErrorString(e), (int)e);
  return ZHA_ERR_HIP;
}

bool valid_refs(int R) { return R == 1 || R == 2 || R == 4 || R == 8 || R == 16; }

// Subtree level of the build: the highest level whose nodes cover at most 256 tokens (>= 1).
int subtree_level(int C, int L) {
  int S = 1;
  int64_t span = C;
  for (int l = 2; l <= L; ++l) {
    span *= C;
    if (span > 256) break;
    S = l;
  }
  return S;
}

zha_status check_desc(const zha_tree_desc* d) {
  if (!d) return ZHA_ERR_INVALID;
  if (d->batch < 1 || d->n_kv_heads < 1 || d->n_q_heads < 1 || d->chunk < 2 || d->levels < 1 || d->n_refs < 1 ||
      d->max_tokens < 1 || d->head_dim < 1)
    return ZHA_ERR_INVALID;
  if (d->dtype != ZHA_F32 && d->dtype != ZHA_BF16) return ZHA_ERR_INVALID;
  if (d->summary != ZHA_SUMMARY_NATIVE && d->summary != ZHA_SUMMARY_FP8 && d->summary != ZHA_SUMMARY_FP4)
    return ZHA_ERR_INVALID;
  if (d->summary != ZHA_SUMMARY_NATIVE && d->dtype != ZHA_BF16) return ZHA_ERR_UNSUPPORTED;
  if (d->n_q_heads % d->n_kv_heads != 0) return ZHA_ERR_INVALID;
  if (d->max_queries < 0) return ZHA_ERR_INVALID;
  {  // routing units of the largest route index the second grid dimension
    const int64_t ru = (int64_t)d->batch * d->n_kv_heads * (d->max_queries > 1 ? d->max_queries : 1) *
                       (d->per_head_routes ? d->n_q_heads / d->n_kv_heads : 1);
    if (ru > 65535) return ZHA_ERR_UNSUPPORTED;
  }
  if (d->batch > ZHA_MAX_BATCH) return ZHA_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return ZHA_ERR_UNSUPPORTED;
  if (!valid_refs(d->n_refs)) return ZHA_ERR_UNSUPPORTED;
  if (d->n_q_heads / d->n_kv_heads > 16) return ZHA_ERR_UNSUPPORTED;
  if (d->levels > ZHA_MAX_LEVELS) return ZHA_ERR_UNSUPPORTED;
  if (d->max_tokens >= ((int64_t)1 << 31)) return ZHA_ERR_UNSUPPORTED;
  if (d->max_tokens / d->chunk >= ((int64_t)1 << 30)) return ZHA_ERR_UNSUPPORTED;
  double span = pow((double)d->chunk, (double)d->levels);
  if (span > (double)(1 << 30)) return ZHA_ERR_UNSUPPORTED;
  const int esize = d->dtype == ZHA_BF16 ? 2 : 4;
  if (zha_build_lds_bytes(d->chunk, subtree_level(d->chunk, d->levels), d->levels, d->head_dim, d->n_refs, esize) >
      160 * 1024)
    return ZHA_ERR_UNSUPPORTED;
  return ZHA_OK;
}

void free_tree(zha_tree* t) {
  if (!t) return;
  for (int l = 0; l < ZHA_MAX_LEVELS + 2; ++l) {
    if (t->m[l]) (void)hipFree(t->m[l]);
    if (t->b[l]) (void)hipFree(t->b[l]);
    if (t->ms[l]) (void)hipFree(t->ms[l]);
    if (t->kept[l]) (void)hipFree(t->kept[l]);
    if (t->krank[l]) (void)hipFree(t->krank[l]);
  }
  void* ps[] = {t->refs,   t->spine,  t->sub_lse, t->sub_m,  t->counts,    t->geo,      t->scores,   t->spart[0], t->spart[1],
                t->sscore[0], t->sscore[1], t->keys,     t->apart,
                t->fh_cnt, t->fh_mass,  t->fh_edge,  t->cut,      t->sel_cand, t->sel_ctr, t->lb_status,
                t->lb_epoch, t->lb_error, t->route_ctr, t->uflag, t->ulist, t->ucount};
  for (void* p : ps)
    if (p) (void)hipFree(p);
  for (int i = 0; i < 2 * ZHA_MAX_TIMING; ++i)
    if (t->ev[i]) (void)hipEventDestroy(t->ev[i]);
  delete t;
}

template <typename P>
bool dalloc(zha_tree* t, P** p, size_t bytes) {
  if (bytes == 0) bytes = 16;
  void* q = nullptr;
  if (hipMalloc(&q, bytes) != hipSuccess) return false;
  *p = (P*)q;
  t->bytes += (int64_t)bytes;
  return true;
}

zha_status check_lens(const zha_tree* t, const int32_t* lens) {
  if (!lens) return ZHA_ERR_INVALID;
  for (int b = 0; b < t->desc.batch; ++b) {
    if (lens[b] < 1) return ZHA_ERR_INVALID;
    if ((int64_t)lens[b] > t->T) return ZHA_ERR_CAPACITY;
  }
  return ZHA_OK;
}

}  // namespace

// ----------------------------------------------------------------------------- timing

static bool zha_timed(const zha_tree* t, int kernel, int level) {
  return (t->timing_kernels >> kernel & 1) && (t->timing_levels >> level & 1) && t->n_rec < ZHA_MAX_TIMING;
}

void zha_time_begin(zha_tree* t, hipStream_t s, int kernel, int level) {
  t->timing_open = zha_timed(t, kernel, level) && hipEventRecord(t->ev[2 * t->n_rec], s) == hipSuccess;
}

void zha_time_end(zha_tree* t, hipStream_t s, int kernel, int level) {
  if (!t->timing_open) return;
  t->timing_open = false;
  if (hipEventRecord(t->ev[2 * t->n_rec + 1], s) != hipSuccess) return;
  t->tk[t->n_rec] = kernel;
  t->tl[t->n_rec] = level;
  ++t->n_rec;
}

extern "C" {

const char* zha_last_error(void) { return g_last_error; }

const char* zha_status_str(zha_status s) {
  switch (s) {
    case ZHA_OK: return "ok";
    case ZHA_ERR_INVALID: return "invalid argument";
    case ZHA_ERR_CAPACITY: return "length exceeds tree capacity";
    case ZHA_ERR_NOMEM: return "out of memory";
    case ZHA_ERR_UNSUPPORTED: return "unsupported shape";
    case ZHA_ERR_HIP: return "HIP runtime error";
    case ZHA_ERR_DEVICE: return "a device-side wait gave up; the routes since the last check are not valid";
  }
  return "unknown status";
}

zha_status zha_tree_create(const zha_tree_desc* desc, zha_tree_t* out) {
  if (!out) return ZHA_ERR_INVALID;
  *out = nullptr;
  zha_status st = check_desc(desc);
  if (st != ZHA_OK) return st;
  zha_tree* t = new (std::nothrow) zha_tree;
  if (!t) return ZHA_ERR_NOMEM;
  memset((void*)t, 0, sizeof(zha_tree));
  t->desc = *desc;
  hipError_t he = hipGetDevice(&t->device);
  if (he != hipSuccess) { delete t; return hip_fail("hipGetDevice", he); }
  t->U = desc->batch * desc->n_kv_heads;
  t->G = desc->n_q_heads / desc->n_kv_heads;
  t->R = desc->n_refs;
  t->d = desc->head_dim;
  t->C = desc->chunk;
  t->L = desc->levels;
  t->T = desc->max_tokens;
  t->esize = desc->dtype == ZHA_BF16 ? 2 : 4;
  t->f8 = desc->summary == ZHA_SUMMARY_FP8;
  t->f4 = desc->summary == ZHA_SUMMARY_FP4;
  const int64_t Nc = (t->T / t->C) * t->C;
  int64_t span = 1;
  for (int l = 1; l <= t->L; ++l) {
    span *= t->C;
    t->span[l] = span;
    t->cap[l] = (Nc + span - 1) / span;
  }
  t->span[0] = 1;
  t->cap[0] = 0;
  const int U = t->U, R = t->R, d = t->d, G = t->G, L = t->L;
  // routing workspace: a route has U * Tq * hr routing units of G / hr heads (Tq queries per
  // sequence up to max_queries; hr = 1, or G with per-head routes); every per-unit array is
  // sized for the largest count, and the per-workgroup partials for the largest product
  const int maxq = desc->max_queries > 1 ? desc->max_queries : 1;
  const int RUmax = U * maxq * (desc->per_head_routes ? G : 1);
  t->RUmax = RUmax;
  t->hr = 1;
  t->Tq = 1;
  t->multi = false;
  t->RU = U;
  t->WS = zha_score_wgs_units(U);
  t->WA = zha_sparse_wgs(U);
  size_t spart_n = 0, apart_n = 0, score_n = 0;
  int64_t cand_n = 0;
  int ctr_n = 0;
  const int hrs[2] = {1, G};
  for (int i = 0; i < (desc->per_head_routes ? 2 : 1); ++i) {
    const int hr = hrs[i], Gr = G / hr;
    for (int tq = 1; tq <= maxq; ++tq) {
      const int ru = U * tq * hr;
      spart_n = std::max(spart_n, (size_t)ru * zha_score_wgs_units(ru) * Gr * 2);
      apart_n = std::max(apart_n, (size_t)ru * zha_sparse_wgs(ru) * Gr * (d + 2));
      score_n = std::max(score_n, (size_t)ru * ((Gr + 3) & ~3));
      cand_n = std::max(cand_n, zha_sel_cand_entries(ru));
      ctr_n = std::max(ctr_n, zha_sel_ctr_words(ru));
      const int ts = zha_union_queries(R, G, tq, hr, desc->dtype == ZHA_BF16);
      const int tss = zha_union_score_queries(R, G, tq, hr);
      if (tss > 0) {  // union scoring: partials of every unit for each workgroup of its group
        const int ng = U * ((tq + tss - 1) / tss);
        spart_n = std::max(spart_n, (size_t)ru * zha_score_wgs_units(ng) * Gr * 2);
      }
      if (ts > 0) {  // union attention: partials of every unit for each workgroup of its group
        const int ng = U * ((tq + ts - 1) / ts);
        apart_n = std::max(apart_n, (size_t)ru * zha_sparse_wgs(ng) * Gr * (d + 2));
      }
    }
  }
  // kept ranks for union routes: some route this tree may serve groups several units
  bool uni = false;
  int ugmax = 0;  // union groups of the largest union route
  for (int i = 0; i < (desc->per_head_routes ? 2 : 1); ++i)
    for (int tq = 1; tq <= maxq; ++tq) {
      const int ts = zha_union_queries(R, G, tq, hrs[i], desc->dtype == ZHA_BF16);
      if (ts > 0) {
        uni = true;
        ugmax = std::max(ugmax, U * ((tq + ts - 1) / ts));
      }
      uni = uni || zha_union_score_queries(R, G, tq, hrs[i]) > 0;
    }
  t->UGmax = ugmax;
  bool ok = true;
  for (int l = 1; l <= L && ok; ++l) {
    const size_t mrow = t->f4 ? (size_t)d / 2 : (size_t)d * (t->f8 ? 1 : t->esize);  // bytes per m row
    ok = ok && dalloc(t, &t->m[l], (size_t)U * t->cap[l] * R * mrow);
    ok = ok && dalloc(t, &t->b[l], (size_t)U * t->cap[l] * R * sizeof(float));
    if (t->f8) ok = ok && dalloc(t, &t->ms[l], (size_t)U * t->cap[l] * R * sizeof(float));
    if (t->f4) ok = ok && dalloc(t, &t->ms[l], (size_t)U * t->cap[l] * R * (d / 32));
    ok = ok && dalloc(t, &t->kept[l], (size_t)RUmax * t->cap[l] * sizeof(int32_t));
    if (uni) ok = ok && dalloc(t, &t->krank[l], (size_t)RUmax * t->cap[l] * sizeof(unsigned long long));
  }
  if (uni) ok = ok && dalloc(t, &t->route_ctr, sizeof(uint32_t));
  ok = ok && dalloc(t, &t->refs, (size_t)desc->n_kv_heads * R * d * sizeof(float));
  ok = ok && dalloc(t, &t->spine, (size_t)U * zha_spine_bytes(L, d, R));
  t->S = subtree_level(t->C, L);
  if (t->S < L) {
    ok = ok && dalloc(t, &t->sub_lse, (size_t)U * t->cap[t->S] * R * sizeof(float));
    ok = ok && dalloc(t, &t->sub_m, (size_t)U * t->cap[t->S] * R * d * sizeof(float));
  }
  ok = ok && dalloc(t, &t->counts, (size_t)2 * (L + 2) * RUmax * sizeof(int32_t));
  ok = ok && dalloc(t, &t->geo, (size_t)(L + 2) * desc->batch * sizeof(int32_t));
  ok = ok && dalloc(t, &t->scores, (size_t)t->cap[1] * score_n * sizeof(float));
  for (int i = 0; i < 2; ++i) {
    ok = ok && dalloc(t, &t->sscore[i], (size_t)zha_small_score_rows() * score_n * sizeof(float));
    ok = ok && dalloc(t, &t->spart[i], spart_n * sizeof(float));
  }
  t->kstride = (t->cap[1] + 3) / 4 * 4;
  ok = ok && dalloc(t, &t->keys, (size_t)RUmax * t->kstride * sizeof(uint32_t));
  if (uni) {
    ok = ok && dalloc(t, &t->uflag, (size_t)ugmax * t->kstride * sizeof(uint32_t));
    ok = ok && dalloc(t, &t->ulist, (size_t)ugmax * t->cap[1] * sizeof(int32_t));
    ok = ok && dalloc(t, &t->ucount, (size_t)2 * ugmax * sizeof(int32_t));
  }
  ok = ok && dalloc(t, &t->apart, apart_n * sizeof(float));
  const int nchunk = zha_compact_chunks(t->cap[1]);
  const int nb = zha_hist_bins();
  ok = ok && dalloc(t, &t->fh_cnt, (size_t)RUmax * nb * sizeof(uint32_t));
  ok = ok && dalloc(t, &t->fh_mass, (size_t)RUmax * nb * sizeof(unsigned long long));
  ok = ok && dalloc(t, &t->fh_edge, (size_t)RUmax * 2 * sizeof(unsigned long long));
  ok = ok && dalloc(t, &t->cut, (size_t)RUmax * 4 * sizeof(int32_t));
  ok = ok && dalloc(t, &t->sel_cand, (size_t)cand_n * 2 * sizeof(uint32_t));
  ok = ok && dalloc(t, &t->sel_ctr, (size_t)ctr_n * sizeof(uint32_t));
  ok = ok && dalloc(t, &t->lb_status, (size_t)RUmax * nchunk * sizeof(unsigned long long));
  ok = ok && dalloc(t, &t->lb_epoch, (size_t)RUmax * 2 * sizeof(uint32_t));
  ok = ok && dalloc(t, &t->lb_error, sizeof(int32_t));
  if (ok) {  // counters and histograms start at zero and are left at zero by the kernels
    ok = hipMemset(t->fh_cnt, 0, (size_t)RUmax * nb * sizeof(uint32_t)) == hipSuccess &&
         hipMemset(t->fh_mass, 0, (size_t)RUmax * nb * sizeof(unsigned long long)) == hipSuccess &&
         hipMemset(t->fh_edge, 0, (size_t)RUmax * 2 * sizeof(unsigned long long)) == hipSuccess &&
         hipMemset(t->sel_ctr, 0, (size_t)ctr_n * sizeof(uint32_t)) == hipSuccess &&
         hipMemset(t->geo, 0, (size_t)(L + 2) * desc->batch * sizeof(int32_t)) == hipSuccess &&
         hipMemset(t->lb_status, 0, (size_t)RUmax * nchunk * sizeof(unsigned long long)) == hipSuccess &&
         hipMemset(t->lb_error, 0, sizeof(int32_t)) == hipSuccess;
    // kept ranks carry the stamp of the route that wrote them; stamps start at 1
    for (int l = 1; l <= L && ok && uni; ++l)
      ok = hipMemset(t->krank[l], 0, (size_t)RUmax * t->cap[l] * sizeof(unsigned long long)) == hipSuccess;
    if (uni) ok = ok && hipMemset(t->route_ctr, 0, sizeof(uint32_t)) == hipSuccess;
    if (uni) ok = ok && hipMemset(t->uflag, 0, (size_t)ugmax * t->kstride * sizeof(uint32_t)) == hipSuccess;
    // union lists start as chunk 0 everywhere, so no entry is ever read before it is written
    if (uni) ok = ok && hipMemset(t->ulist, 0, (size_t)ugmax * t->cap[1] * sizeof(int32_t)) == hipSuccess;
    // every unit's epoch starts at 1: status words of epoch 0 (all-zero memory) never match
    std::vector<uint32_t> ep((size_t)RUmax * 2, 0u);
    for (int u = 0; u < RUmax; ++u) ep[(size_t)u * 2] = 1u;
    ok = ok && hipMemcpy(t->lb_epoch, ep.data(), ep.size() * sizeof(uint32_t), hipMemcpyHostToDevice) == hipSuccess;
    ok = ok && hipDeviceSynchronize() == hipSuccess;
  }
  if (!ok) {
    free_tree(t);
    return ZHA_ERR_NOMEM;
  }
  *out = t;
  return ZHA_OK;
}

void zha_tree_destroy(zha_tree_t t) { free_tree(t); }

zha_status zha_tree_bytes(zha_tree_t t, int64_t* bytes) {
  if (!t || !bytes) return ZHA_ERR_INVALID;
  *bytes = t->bytes;
  return ZHA_OK;
}

zha_status zha_build(zha_tree_t t, const void* K, const float* refs, const int32_t* seq_lens, hipStream_t s) {
  if (!t || !K || !refs) return ZHA_ERR_INVALID;
  zha_status st = check_lens(t, seq_lens);
  if (st != ZHA_OK) return st;
  for (int b = 0; b < t->desc.batch; ++b) t->len.n[b] = seq_lens[b];
  t->len_prev = t->len;
  hipError_t e = hipMemcpyAsync(t->refs, refs, (size_t)t->desc.n_kv_heads * t->R * t->d * sizeof(float),
                                hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) return hip_fail("zha_build copy of refs", e);
  e = zha_launch_build(t, K, s);
  if (e != hipSuccess) return hip_fail("zha_build launch", e);
  t->built = true;
  ++t->gen;
  return ZHA_OK;
}

zha_status zha_append(zha_tree_t t, const void* K, const int32_t* new_seq_lens, hipStream_t s) {
  if (!t || !K) return ZHA_ERR_INVALID;
  if (!t->built) return ZHA_ERR_INVALID;
  zha_status st = check_lens(t, new_seq_lens);
  if (st != ZHA_OK) return st;
  for (int b = 0; b < t->desc.batch; ++b)
    if (new_seq_lens[b] < t->len.n[b]) return ZHA_ERR_INVALID;
  t->len_prev = t->len;
  for (int b = 0; b < t->desc.batch; ++b) t->len.n[b] = new_seq_lens[b];
  ++t->gen;  // the lengths changed: the last route's kept lists are stale from here on
  hipError_t e = zha_launch_append(t, K, s);
  if (e != hipSuccess) return hip_fail("zha_append launch", e);
  return ZHA_OK;
}

// A route of Tq queries per sequence (multi: a block of queries, whose attention also reads
// the block's own rows).
static zha_status route_queries(zha_tree* t, const void* q, int Tq, bool multi, float p, float scale,
                                zha_route_mode mode, zha_kept* kept, hipStream_t s) {
  if (!t || !q || !kept) return ZHA_ERR_INVALID;
  if (!t->built) return ZHA_ERR_INVALID;
  if (!(p > 0.0f) || !isfinite(p) || !isfinite(scale)) return ZHA_ERR_INVALID;
  if (mode != ZHA_ROUTE_GROUP && mode != ZHA_ROUTE_PER_HEAD) return ZHA_ERR_INVALID;
  if (mode == ZHA_ROUTE_PER_HEAD && !t->desc.per_head_routes) return ZHA_ERR_INVALID;
  if (Tq < 1) return ZHA_ERR_INVALID;
  if (Tq > (t->desc.max_queries > 1 ? t->desc.max_queries : 1)) return ZHA_ERR_CAPACITY;
  t->hr = mode == ZHA_ROUTE_PER_HEAD ? t->G : 1;
  t->Tq = Tq;
  t->multi = multi;
  t->RU = t->U * Tq * t->hr;
  t->WS = zha_score_wgs_units(t->RU);
  t->WA = zha_sparse_wgs(t->RU);
  t->route_gen = t->gen;
  hipError_t e = zha_launch_route(t, q, p, scale, s);
  if (e != hipSuccess) return hip_fail("zha_route launch", e);
  kept->counts = t->counts + (int64_t)(t->L + 2) * t->RU + t->RU;
  kept->ids = t->kept[1];
  kept->cap = t->cap[1];
  return ZHA_OK;
}

zha_status zha_route_ex(zha_tree_t t, const void* q, float p, float scale, zha_route_mode mode, zha_kept* kept,
                        hipStream_t s) {
  return route_queries(t, q, 1, false, p, scale, mode, kept, s);
}

zha_status zha_route_multi(zha_tree_t t, const void* q, int32_t n_queries, float p, float scale,
                           zha_route_mode mode, zha_kept* kept, hipStream_t s) {
  return route_queries(t, q, n_queries, true, p, scale, mode, kept, s);
}

zha_status zha_route(zha_tree_t t, const void* q, float p, float scale, zha_kept* kept, hipStream_t s) {
  return zha_route_ex(t, q, p, scale, ZHA_ROUTE_GROUP, kept, s);
}

zha_status zha_attend(zha_tree_t t, const void* q, const void* K, const void* V, const zha_kept* kept, float scale,
                      float* out, float* lse, hipStream_t s) {
  if (!t || !q || !K || !V || !kept || !out || !lse) return ZHA_ERR_INVALID;
  if (!t->built) return ZHA_ERR_INVALID;
  if (kept->ids != t->kept[1]) return ZHA_ERR_INVALID;  // a view of this tree's last route
  if (t->route_gen != t->gen) return ZHA_ERR_INVALID;   // built or appended to since that route
  if (t->multi) return ZHA_ERR_INVALID;                 // a block of queries: zha_attend_multi
  if (!isfinite(scale)) return ZHA_ERR_INVALID;
  hipError_t e = zha_launch_attend(t, q, K, V, scale, out, lse, s);
  if (e != hipSuccess) return hip_fail("zha_attend launch", e);
  return ZHA_OK;
}

zha_status zha_attend_multi(zha_tree_t t, const void* q, int32_t n_queries, const void* K, const void* V,
                            const zha_kept* kept, float scale, float* out, float* lse, hipStream_t s) {
  if (!t || !q || !K || !V || !kept || !out || !lse) return ZHA_ERR_INVALID;
  if (!t->built) return ZHA_ERR_INVALID;
  if (kept->ids != t->kept[1]) return ZHA_ERR_INVALID;
  if (t->route_gen != t->gen) return ZHA_ERR_INVALID;           // built or appended to since that route
  if (!t->multi || n_queries != t->Tq) return ZHA_ERR_INVALID;  // the last route carried this block
  if (!isfinite(scale)) return ZHA_ERR_INVALID;
  for (int b = 0; b < t->desc.batch; ++b)  // the block's rows N .. N + Tq - 1 lie inside K and V
    if ((int64_t)t->len.n[b] + n_queries > t->T) return ZHA_ERR_CAPACITY;
  hipError_t e = zha_launch_attend(t, q, K, V, scale, out, lse, s);
  if (e != hipSuccess) return hip_fail("zha_attend_multi launch", e);
  return ZHA_OK;
}

zha_status zha_tree_check(zha_tree_t t, hipStream_t s) {
  if (!t) return ZHA_ERR_INVALID;
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail("zha_tree_check synchronize", e);
  int32_t flag = 0;
  e = hipMemcpy(&flag, t->lb_error, sizeof(int32_t), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail("zha_tree_check read", e);
  if (flag == 0) return ZHA_OK;
  e = hipMemset(t->lb_error, 0, sizeof(int32_t));
  if (e != hipSuccess) return hip_fail("zha_tree_check clear", e);
  e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail("zha_tree_check clear", e);
  return ZHA_ERR_DEVICE;
}

size_t zha_dense_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                 int64_t max_tokens) {
  (void)max_tokens;
  if (batch < 1 || n_kv_heads < 1 || n_q_heads < n_kv_heads || head_dim < 1) return 0;
  const int U = batch * n_kv_heads;
  return (size_t)U * zha_dense_wgs(U) * (n_q_heads / n_kv_heads) * (head_dim + 2) * sizeof(float);
}

}  // extern "C"

// Split-K partials of zha_dense_decode_noalloc: one array per GPU, held until the process
// ends.  Host code never passes `scratch` itself to a kernel (on the host it names a
// stand-in, not device memory): the device address is taken once per device with
// hipGetSymbolAddress, with that device current, and kept in g_scratch.
static __device__ __align__(256) float scratch[ZHA_DENSE_SCRATCH_BYTES / sizeof(float)];

namespace {
constexpr int ZHA_MAX_DEVICES = 256;
std::mutex g_scratch_mu;
void* g_scratch[ZHA_MAX_DEVICES];

// The current device's address of `scratch` (taken on the first call on that device).
zha_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("zha_dense_decode_noalloc hipGetDevice", e);
  if (dev < 0 || dev >= ZHA_MAX_DEVICES) return ZHA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail("zha_dense_decode_noalloc hipGetSymbolAddress", e);
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return ZHA_OK;
}

// Validation and launch of dense decode; workspace null: the partials go to the device's
// scratch array (checked to fit before anything touches the device).
zha_status dense_decode_impl(const void* q, const void* K, const void* V, const int32_t* seq_lens, int32_t batch,
                             int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int64_t max_tokens,
                             zha_dtype dtype, float scale, float* out, float* lse, void* workspace,
                             size_t workspace_bytes, bool noalloc, hipStream_t s) {
  if (!q || !K || !V || !seq_lens || !out || !lse || (!noalloc && !workspace)) return ZHA_ERR_INVALID;
  if (batch < 1 || n_kv_heads < 1 || n_q_heads < 1 || n_q_heads % n_kv_heads != 0 || max_tokens < 1)
    return ZHA_ERR_INVALID;
  if (dtype != ZHA_F32 && dtype != ZHA_BF16) return ZHA_ERR_INVALID;
  if (!isfinite(scale)) return ZHA_ERR_INVALID;
  if (batch > ZHA_MAX_BATCH || (head_dim != 64 && head_dim != 128) || n_q_heads / n_kv_heads > 16 ||
      max_tokens >= ((int64_t)1 << 31))
    return ZHA_ERR_UNSUPPORTED;
  const size_t need = zha_dense_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, max_tokens);
  if (noalloc && need > ZHA_DENSE_SCRATCH_BYTES) return ZHA_ERR_CAPACITY;
  if (!noalloc && workspace_bytes < need) return ZHA_ERR_INVALID;
  ZLens len;
  memset(&len, 0, sizeof(len));
  for (int b = 0; b < batch; ++b) {
    if (seq_lens[b] < 1) return ZHA_ERR_INVALID;
    if ((int64_t)seq_lens[b] > max_tokens) return ZHA_ERR_CAPACITY;
    len.n[b] = seq_lens[b];
  }
  if (noalloc) {
    const zha_status st = scratch_address(&workspace);
    if (st != ZHA_OK) return st;
  }
  const int U = batch * n_kv_heads;
  hipError_t e = zha_launch_dense(q, K, V, len, batch, n_q_heads, n_kv_heads, head_dim, max_tokens, dtype, scale,
                                  out, lse, (float*)workspace, zha_dense_wgs(U), s);
  if (e != hipSuccess) return hip_fail(noalloc ? "zha_dense_decode_noalloc launch" : "zha_dense_decode launch", e);
  return ZHA_OK;
}
}  // namespace

extern "C" {

zha_status zha_dense_decode(const void* q, const void* K, const void* V, const int32_t* seq_lens, int32_t batch,
                            int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int64_t max_tokens,
                            zha_dtype dtype, float scale, float* out, float* lse, void* workspace,
                            size_t workspace_bytes, hipStream_t s) {
  return dense_decode_impl(q, K, V, seq_lens, batch, n_q_heads, n_kv_heads, head_dim, max_tokens, dtype, scale, out,
                           lse, workspace, workspace_bytes, false, s);
}

zha_status zha_dense_decode_noalloc(const void* q, const void* K, const void* V, const int32_t* seq_lens,
                                    int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                    int64_t max_tokens, zha_dtype dtype, float scale, float* out, float* lse,
                                    hipStream_t s) {
  return dense_decode_impl(q, K, V, seq_lens, batch, n_q_heads, n_kv_heads, head_dim, max_tokens, dtype, scale, out,
                           lse, nullptr, 0, true, s);
}

zha_status zha_tree_level_capacity(zha_tree_t t, int32_t level, int64_t* nodes) {
  if (!t || !nodes || level < 1 || level > t->L) return ZHA_ERR_INVALID;
  *nodes = t->cap[level];
  return ZHA_OK;
}

zha_status zha_tree_copy_level(zha_tree_t t, int32_t level, void* m_out, float* b_out, hipStream_t s) {
  if (!t || !m_out || !b_out || level < 1 || level > t->L) return ZHA_ERR_INVALID;
  const size_t nm = (size_t)t->U * t->cap[level] * t->R;
  if (t->f8) {
    const hipError_t e = zha_launch_decode_fp8((const uint8_t*)t->m[level], t->ms[level], (int64_t)nm, t->d,
                                               (__bf16*)m_out, s);
    if (e != hipSuccess) return hip_fail("zha_tree_copy_level", e);
  } else if (t->f4) {
    const hipError_t e = zha_launch_decode_fp4((const uint8_t*)t->m[level], (const uint8_t*)t->ms[level], (int64_t)nm,
                                               t->d, (__bf16*)m_out, nullptr, s);
    if (e != hipSuccess) return hip_fail("zha_tree_copy_level", e);
  } else if (hipMemcpyAsync(m_out, t->m[level], nm * t->d * t->esize, hipMemcpyDeviceToDevice, s) != hipSuccess) {
    return ZHA_ERR_HIP;
  }
  if (hipMemcpyAsync(b_out, t->b[level], nm * sizeof(float), hipMemcpyDeviceToDevice, s) != hipSuccess)
    return ZHA_ERR_HIP;
  return ZHA_OK;
}

zha_status zha_tree_copy_scales(zha_tree_t t, int32_t level, float* scale_out, hipStream_t s) {
  if (!t || !scale_out || level < 1 || level > t->L || !(t->f8 || t->f4)) return ZHA_ERR_INVALID;
  const size_t nm = (size_t)t->U * t->cap[level] * t->R;
  if (t->f4) {
    const hipError_t e = zha_launch_decode_fp4((const uint8_t*)t->m[level], (const uint8_t*)t->ms[level], (int64_t)nm,
                                               t->d, nullptr, scale_out, s);
    return e == hipSuccess ? ZHA_OK : hip_fail("zha_tree_copy_scales", e);
  }
  if (hipMemcpyAsync(scale_out, t->ms[level], nm * sizeof(float), hipMemcpyDeviceToDevice, s) != hipSuccess)
    return ZHA_ERR_HIP;
  return ZHA_OK;
}

zha_status zha_route_copy_level(zha_tree_t t, int32_t level, int32_t* frontier_counts, int32_t* kept_counts,
                                int32_t* kept_ids, hipStream_t s) {
  if (!t || !frontier_counts || !kept_counts || !kept_ids || level < 1 || level > t->L) return ZHA_ERR_INVALID;
  const int U = t->RU;  // routing units of the last route
  const int32_t* cF = t->counts + (int64_t)level * U;
  const int32_t* cK = t->counts + (int64_t)(t->L + 2) * U + (int64_t)level * U;
  if (hipMemcpyAsync(frontier_counts, cF, U * sizeof(int32_t), hipMemcpyDeviceToDevice, s) != hipSuccess ||
      hipMemcpyAsync(kept_counts, cK, U * sizeof(int32_t), hipMemcpyDeviceToDevice, s) != hipSuccess ||
      hipMemcpyAsync(kept_ids, t->kept[level], (size_t)U * t->cap[level] * sizeof(int32_t), hipMemcpyDeviceToDevice,
                     s) != hipSuccess)
    return ZHA_ERR_HIP;
  return ZHA_OK;
}

zha_status zha_timing_enable(zha_tree_t t, int32_t kernel_mask, int32_t level_mask) {
  if (!t) return ZHA_ERR_INVALID;
  if (kernel_mask && !t->ev[0]) {
    // timing-only events: no system-scope fence when recorded (the writeback and invalidation
    // of the caches that fence costs would sit between the timed launch and its neighbours)
    for (int i = 0; i < 2 * ZHA_MAX_TIMING; ++i)
      if (hipEventCreateWithFlags(&t->ev[i], hipEventDisableSystemFence) != hipSuccess) return ZHA_ERR_HIP;
  }
  t->timing_kernels = kernel_mask;
  t->timing_levels = level_mask;
  t->timing_open = false;
  return ZHA_OK;
}

zha_status zha_timing_read(zha_tree_t t, int32_t* kernels, int32_t* levels, float* ms, int32_t max_entries,
                           int32_t* n_entries) {
  if (!t || !n_entries || max_entries < 0 || (max_entries > 0 && (!kernels || !levels || !ms)))
    return ZHA_ERR_INVALID;
  const int n = t->n_rec < max_entries ? t->n_rec : max_entries;
  for (int i = 0; i < n; ++i) {
    float x = 0.0f;
    if (hipEventElapsedTime(&x, t->ev[2 * i], t->ev[2 * i + 1]) != hipSuccess) return ZHA_ERR_HIP;
    kernels[i] = t->tk[i];
    levels[i] = t->tl[i];
    ms[i] = x;
  }
  *n_entries = n;
  t->n_rec = 0;
  return ZHA_OK;
}

zha_status zha_calibration_copy(void* dst, const void* src, int64_t n16, hipStream_t s) {
  if (!dst || !src || n16 < 0) return ZHA_ERR_INVALID;
  if (((uintptr_t)dst & 15) || ((uintptr_t)src & 15)) return ZHA_ERR_INVALID;
  hipError_t e = zha_launch_copy16(dst, src, n16, s);
  if (e != hipSuccess) return hip_fail("zha_calibration_copy launch", e);
  return ZHA_OK;
}

}  // extern "C"
