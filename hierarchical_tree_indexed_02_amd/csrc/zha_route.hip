// zha_route.hip -- top-down routing of the decode queries through the summary tree.
//
// Method ([wqu] "How does top-p routing pick tokens?"; page key in include/zha.h):
// at each level the frontier nodes are scored, the smallest set holding a
// fraction p of the estimated attention mass is kept, and only the kept
// nodes' children form the next frontier.  A node's score for a query head is
// the maximum of its reference queries' tangent planes, b_r + scale * q.m_r
// ([wqu] "Building the tree").  The G query heads of one KV head share one kept
// set: a node's mass is the mean over the heads of its frontier-normalised mass.
//
// Kernels of one level (U = sequences x KV heads, the "units"):
//   zha_score_kernel    many workgroups per unit stream the frontier's planes from
//                       HBM once and score them on the matrix cores (G query heads x
//                       R planes per node is a small dense product), and write the
//                       per-workgroup (max, sum exp) partials of each head's scores.
//   small frontiers (<= 4096 nodes): zha_select_small_kernel, one workgroup per unit,
//                       forms the node masses, finds the exact cut and compacts, in LDS.
//   large frontiers:    zha_mass_kernel (many workgroups) forms the masses and an exact
//                       histogram of them on fixed slices around the uniform mass 1/|F|;
//                       zha_select_large_kernel (one workgroup per unit) resolves the cut
//                       from the histogram and the few keys of the crossing slice;
//                       zha_compact_kernel (many workgroups) writes the kept ids in order,
//                       chaining chunk offsets with a decoupled look-back.
// The cut: nodes ordered by (mass descending, id ascending); keep the shortest
// prefix whose mass reaches p times the frontier's total.  Masses are compared as
// fp32 bit patterns ("keys") and summed as 40-bit fixed-point integers, so every
// sum is exact and independent of order: results are bit-identical run to run.
#include "zha_internal.h"

namespace {

typedef unsigned long long u64;

constexpr int NB = 1024;                 // histogram slices
constexpr int SMALL_NODES = 4096;        // frontiers up to this size are selected in LDS
constexpr int CAND = 8192;               // keys of a crossing slice held in LDS
constexpr int CH = 1024;                 // compaction chunk (positions per workgroup)

// Per-level inputs shared by the kernels of one level.
struct Level {
  const int32_t* parent;      // kept ids of level l+1 [U][cap_parent]; null at the top level
  const int32_t* parent_nF;   // frontier counts of this level, written by level l+1 [U]
  int64_t cap_parent;
  int64_t span_l;             // tokens per node at this level, C^l
  int C, Cshift, Hkv;
  ZLens len;
};

__device__ __forceinline__ int frontier_size(const Level& v, int u) {
  if (v.parent) return v.parent_nF[u];
  const int64_t N = v.len.n[u / v.Hkv];
  const int64_t Nc = (N / v.C) * v.C;
  return (int)((Nc + v.span_l - 1) / v.span_l);
}

// Node id of frontier position pos: the top level lists every node; a lower level
// lists the children of the kept parents in order (only the last parent can be partial).
__device__ __forceinline__ int frontier_id(const int32_t* par, int pos, int C, int Cshift) {
  if (!par) return pos;
  if (Cshift >= 0) return (par[pos >> Cshift] << Cshift) + (pos & ((1 << Cshift) - 1));
  const int k = pos / C;
  return par[k] * C + (pos - k * C);
}

// Frontier size of the next level given this level's kept count and last kept id.
__device__ __forceinline__ int next_frontier(int kept, int last_id, int C, int n_child) {
  if (kept == 0) return 0;
  return C * (kept - 1) + min(C, n_child - last_id * C);
}

__device__ __forceinline__ int child_nodes(const Level& v, int u, int64_t span_child) {
  const int64_t N = v.len.n[u / v.Hkv];
  const int64_t Nc = (N / v.C) * v.C;
  return (int)((Nc + span_child - 1) / span_child);
}

__device__ __forceinline__ void lse_push(float& M, float& S, float x) {
  if (x == -INFINITY) return;
  if (x > M) {
    S = S * zexp(M - x) + 1.0f;
    M = x;
  } else {
    S += zexp(x - M);
  }
}

__device__ __forceinline__ void lse_merge(float& M, float& S, float M2, float S2) {
  const float mx = fmaxf(M, M2);
  if (mx == -INFINITY) { M = -INFINITY; S = 0.0f; return; }
  S = S * zexp(M - mx) + S2 * zexp(M2 - mx);
  M = mx;
}

// Fixed-point mass of a key: w * 2^40 truncated (w <= 1 up to rounding).
__device__ __forceinline__ u64 fx_mass(uint32_t key) { return (u64)(__uint_as_float(key) * 1099511627776.0f); }

// Node mass key from its G scores: mean over heads of exp(s_h - LSE_h), as fp32 bits.
__device__ __forceinline__ uint32_t mass_key(const float (&sv)[16], const float* lse, int G, float invG) {
  float w = 0.0f;
#pragma unroll
  for (int h = 0; h < 16; ++h)
    if (h < G) w += zexp(sv[h] - lse[h]);
  return __float_as_uint(w * invG);
}

__device__ __forceinline__ void load_scores(const float* sp, int G, bool valid, float (&sv)[16]) {
  if ((G & 3) == 0) {  // a node's G scores are 16-byte aligned
#pragma unroll
    for (int h4 = 0; h4 < 4; ++h4) {
      const float4 v = (valid && 4 * h4 < G) ? *(const float4*)(sp + 4 * h4) : make_float4(0.f, 0.f, 0.f, 0.f);
      sv[4 * h4] = v.x; sv[4 * h4 + 1] = v.y; sv[4 * h4 + 2] = v.z; sv[4 * h4 + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int h = 0; h < 16; ++h) sv[h] = (valid && h < G) ? sp[h] : 0.0f;
  }
}

// ----------------------------------------------------------------------------------- score

struct ScoreArgs {
  Level v;
  const void* m;          // level planes m [U][capl][R][d]
  const float* b;         // level planes b [U][capl][R]
  const void* q;          // [B][Hq][d]
  int64_t capl;
  float* scores;          // [U][cap1][G]
  int64_t cap1;
  float* part;            // [U][W][G][2]: (max, sum exp) of the workgroup's scores per head
  int W;                  // workgroups per unit
  int Hq, G;
  float scale;
};

// Scores one level's frontier.  Rows of an MFMA tile are (node, reference query)
// pairs: 16/R nodes per tile; columns are the KV head's query heads (G <= 16).
// Lane i loads its row's plane slice (k-slot group i/16) straight from HBM; the
// query fragments stay in registers for the whole workgroup.
template <typename T, int R, int D, int UN>
__global__ __launch_bounds__(256) void zha_score_kernel(ScoreArgs a) {
  typedef Mf<T> M;
  constexpr int NK = D / M::KPER;
  constexpr int NPT = 16 / R;
  constexpr int SUPER = 4 * UN * NPT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane & 15, grp = lane >> 4;
  const int u = blockIdx.y, bi = u / a.v.Hkv, g = u % a.v.Hkv;
  const int G = a.G;
  const int nF = frontier_size(a.v, u);
  int per = (nF + a.W - 1) / a.W;
  per = ((per + SUPER - 1) / SUPER) * SUPER;
  const int start = blockIdx.x * per;
  const int end = min(nF, start + per);

  typename M::frag qf[NK];
  {
    const T* qp = (const T*)a.q + ((int64_t)bi * a.Hq + (int64_t)g * G + row) * D + grp * M::EPL;
#pragma unroll
    for (int s = 0; s < NK; ++s) qf[s] = row < G ? M::load(qp + s * M::KPER) : M::zero();
  }
  const int32_t* par = a.v.parent ? a.v.parent + (int64_t)u * a.v.cap_parent : nullptr;
  const T* mb = (const T*)a.m + (int64_t)u * a.capl * R * D;
  const float* bb = a.b + (int64_t)u * a.capl * R;
  float* sc = a.scores + (int64_t)u * a.cap1 * G;
  float runM = -INFINITY, runS = 0.0f;

  for (int base = start; base < end; base += SUPER) {
    typename M::frag af[UN][NK];
    float bv[UN][4];
    int tb[UN];
#pragma unroll
    for (int k = 0; k < UN; ++k) {
      tb[k] = base + (k * 4 + wave) * NPT;
      const int pos = tb[k] + row / R;
      const bool v = pos < end;
      const int id = v ? frontier_id(par, pos, a.v.C, a.v.Cshift) : 0;
      const T* mp = mb + ((int64_t)id * R + (row % R)) * D + grp * M::EPL;
#pragma unroll
      for (int s = 0; s < NK; ++s) af[k][s] = v ? M::load(mp + s * M::KPER) : M::zero();
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r2 = 4 * grp + jj;
        const int id2 = __shfl(id, r2);
        const bool v2 = tb[k] + r2 / R < end;
        bv[k][jj] = v2 ? bb[(int64_t)id2 * R + (r2 % R)] : -INFINITY;
      }
    }
#pragma unroll
    for (int k = 0; k < UN; ++k) {
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < NK; ++s) acc = M::mma(af[k][s], qf[s], acc);
      float v[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) v[jj] = bv[k][jj] == -INFINITY ? -INFINITY : fmaf(acc[jj], a.scale, bv[k][jj]);
      // maximum over each node's planes; rows 4*grp+jj of this lane belong to node (4*grp+jj)/R
      if (R >= 4) {
        float mx = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
        if (R >= 8) mx = fmaxf(mx, __shfl_xor(mx, 16));
        if (R >= 16) mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool writer = (R == 4) || (R == 8 && (grp & 1) == 0) || (R == 16 && grp == 0);
        const int pos = tb[k] + (4 * grp) / R;
        if (writer && row < G && pos < end) {
          sc[(int64_t)pos * G + row] = mx;
          lse_push(runM, runS, mx);
        }
      } else if (R == 2) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const float mx = fmaxf(v[2 * h2], v[2 * h2 + 1]);
          const int pos = tb[k] + 2 * grp + h2;
          if (row < G && pos < end) {
            sc[(int64_t)pos * G + row] = mx;
            lse_push(runM, runS, mx);
          }
        }
      } else {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int pos = tb[k] + 4 * grp + jj;
          if (row < G && pos < end) {
            sc[(int64_t)pos * G + row] = v[jj];
            lse_push(runM, runS, v[jj]);
          }
        }
      }
    }
  }
  // per-head (max, sum exp) of this workgroup: lanes of one head, then the 4 waves
  {
    float M2 = __shfl_xor(runM, 16), S2 = __shfl_xor(runS, 16);
    lse_merge(runM, runS, M2, S2);
    M2 = __shfl_xor(runM, 32);
    S2 = __shfl_xor(runS, 32);
    lse_merge(runM, runS, M2, S2);
  }
  __shared__ float sM[4][16], sS[4][16];
  if (grp == 0) { sM[wave][row] = runM; sS[wave][row] = runS; }
  __syncthreads();
  if (threadIdx.x < G) {
    float Mx = sM[0][threadIdx.x], Sx = sS[0][threadIdx.x];
    for (int w = 1; w < 4; ++w) lse_merge(Mx, Sx, sM[w][threadIdx.x], sS[w][threadIdx.x]);
    float* pp = a.part + (((int64_t)u * a.W + blockIdx.x) * G + threadIdx.x) * 2;
    pp[0] = Mx;
    pp[1] = Sx;
  }
}

// Per-head log-sum-exp over the frontier from the W scoring partials of unit u, into
// lse[0..G).  Heads go to groups of 16 threads; each group combines the partials in a
// fixed order, so every workgroup that calls this gets the same bits.
template <int NT>
__device__ __forceinline__ void frontier_lse(const float* part, int W, int G, int u, float* lse) {
  static_assert(NT >= 256, "16 threads per head for up to 16 heads");
  const int h = threadIdx.x >> 4, j = threadIdx.x & 15;
  float Mx = -INFINITY, Sx = 0.0f;
  if (h < G) {
    for (int i0 = j; i0 < W; i0 += 16 * 8) {
      float2 pv[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int i = i0 + 16 * k;
        pv[k] = i < W ? *(const float2*)(part + (((int64_t)u * W + i) * G + h) * 2) : make_float2(-INFINITY, 0.0f);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) lse_merge(Mx, Sx, pv[k].x, pv[k].y);
    }
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) {
    const float M2 = __shfl_xor(Mx, o, 16), S2 = __shfl_xor(Sx, o, 16);
    lse_merge(Mx, Sx, M2, S2);
  }
  if (h < G && j == 0) lse[h] = Mx + zlog(Sx);
}

// ------------------------------------------------------------------------ shared selection

// Exclusive scan of one u32 per thread over a workgroup of NT threads; total in *tot.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* tot, uint32_t* sh) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  uint32_t before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t c = sh[w];
    if (w < wave) before += c;
    total += c;
  }
  *tot = total;
  __syncthreads();
  return before + inc - x;
}

// Given an NB-bin histogram of fixed-point masses and the mass already above the bins,
// find the bin in which the cumulative mass, from the heaviest bin down, reaches T.
// One wave; lane l owns NB/64 consecutive bins from the top.  Writes only when found.
__device__ __forceinline__ void find_bin(const u64* hm, u64 above0, u64 T, uint32_t* out_bin, u64* out_above) {
  constexpr int PER = NB / 64;
  const int lane = threadIdx.x & 63;
  u64 ls = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) ls += hm[NB - 1 - PER * lane - e];
  u64 inc = ls;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const u64 y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  u64 run = above0 + inc - ls;
  if (run < T && run + ls >= T) {
    for (int e = 0; e < PER; ++e) {
      const int bin = NB - 1 - PER * lane - e;
      const u64 m = hm[bin];
      if (run < T && run + m >= T) {
        *out_bin = (uint32_t)bin;
        *out_above = run;
        break;
      }
      run += m;
    }
  }
}

// Bin of `key` among NB equal slices of the integer key range [lo, lo + span); monotone in key.
__device__ __forceinline__ uint32_t range_bin(uint32_t key, uint32_t lo, u64 span) {
  return (uint32_t)(((u64)(key - lo) * (u64)NB) / span);
}

// Key range of slice b of [lo, lo + span).
__device__ __forceinline__ void slice_range(uint32_t lo, u64 span, uint32_t b, uint32_t* nlo, uint32_t* nhi) {
  *nlo = lo + (uint32_t)(((u64)b * span + NB - 1) / NB);
  *nhi = lo + (uint32_t)((((u64)b + 1) * span + NB - 1) / NB) - 1;
}

// Key window of the fine histogram: 20 binades of fp32 around the uniform mass 1/n
// (from 2^-16/n to 16/n), cut in NB slices of 1/51 binade.
__device__ __forceinline__ void fine_window(int n, uint32_t* lo, u64* span) {
  const uint32_t ref = __float_as_uint(1.0f / (float)n);
  *lo = ref - (16u << 23);
  *span = (u64)20 << 23;
}

// Selection state of one workgroup (LDS).
template <int NT>
struct SelSh {
  uint32_t ckey[CAND];
  uint32_t cpos[CAND];
  uint32_t hcnt[NB];
  u64 hmass[NB];
  u64 red64[2 * (NT / 64)];
  uint32_t scan[NT / 64];
  uint32_t bin, ncand, neq;
  int lastpos;
  u64 above, T;
};

template <int NT>
__device__ __forceinline__ void hist_clear(SelSh<NT>& sh) {
  for (int i = threadIdx.x; i < NB; i += NT) { sh.hcnt[i] = 0; sh.hmass[i] = 0; }
}

template <int NT>
__device__ __forceinline__ u64 block_sum_u64(u64 x, u64* red) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  __syncthreads();
  if (lane == 0) red[wave] = x;
  __syncthreads();
  u64 t = 0;
  for (int w = 0; w < NW; ++w) t += red[w];
  return t;
}

// Histogram of keys[0, n) over the slices of [lo, lo + span) (keys outside are skipped).
template <int NT>
__device__ __forceinline__ void hist_keys(SelSh<NT>& sh, const uint32_t* keys, int n, uint32_t lo, u64 span) {
  const uint32_t hi = (uint32_t)((u64)lo + span - 1);
  for (int i = threadIdx.x; i < n; i += NT) {
    const uint32_t k = keys[i];
    if (k >= lo && k <= hi) {
      const uint32_t bn = range_bin(k, lo, span);
      atomicAdd(&sh.hcnt[bn], 1u);
      atomicAdd(&sh.hmass[bn], fx_mass(k));
    }
  }
}

// With sh.hmass a histogram of [lo, lo + span) holding the cut and sh.above the mass of
// every key above the range, refine NB-fold per step over keys[0, n) until one key value
// remains.  Returns tau; sh.above ends as the mass of the keys above tau.
template <int NT>
__device__ __forceinline__ uint32_t refine_cut(SelSh<NT>& sh, const uint32_t* keys, int n, uint32_t lo, u64 span,
                                               u64 T) {
  const int wave = threadIdx.x >> 6;
  if (wave == 0) find_bin(sh.hmass, sh.above, T, &sh.bin, &sh.above);
  __syncthreads();
  uint32_t nlo, nhi;
  slice_range(lo, span, sh.bin, &nlo, &nhi);
  while (nhi > nlo) {
    const uint32_t l2 = nlo;
    const u64 s2 = (u64)nhi - nlo + 1;
    __syncthreads();
    hist_clear(sh);
    __syncthreads();
    hist_keys<NT>(sh, keys, n, l2, s2);
    __syncthreads();
    if (wave == 0) find_bin(sh.hmass, sh.above, T, &sh.bin, &sh.above);
    __syncthreads();
    slice_range(l2, s2, sh.bin, &nlo, &nhi);
  }
  return nlo;
}

// Ties at the cut all carry the same mass: the fewest that reach T.
__device__ __forceinline__ uint32_t ties_to_take(uint32_t tau, u64 T, u64 above) {
  const u64 mt = fx_mass(tau) > 0 ? fx_mass(tau) : 1;  // the cut element always carries mass
  return (uint32_t)((T - above + mt - 1) / mt);
}

__device__ __forceinline__ u64 target_of(float p, u64 total) {
  u64 T = (u64)ceil((double)p * (double)total);  // c >= p W  <=>  c >= ceil(p W) for integer c
  if (T < 1) T = 1;
  if (T > total) T = total;
  return T;
}

// --------------------------------------------------------------------------- small levels

struct SmallArgs {
  Level v;
  const float* scores;    // [U][cap1][G]
  int64_t cap1;
  const float* part;      // [U][W][G][2] scoring partials
  int W;
  int32_t* kept;          // [U][capl]
  int64_t capl;
  int32_t* nF_out;        // this level's frontier counts [U]
  int32_t* kept_count;    // [U]
  int32_t* next_nF;       // next level's frontier counts [U]; null at level 1
  int64_t span_child;     // C^(l-1)
  int G;
  float p;
  int keep_all;
};

constexpr int SMT = 256;  // threads of the small-level selection

// Whole selection of a frontier of at most SMALL_NODES nodes in one workgroup, in LDS.
__global__ __launch_bounds__(SMT) void zha_select_small_kernel(SmallArgs a) {
  __shared__ uint32_t s_keys[SMALL_NODES];
  __shared__ SelSh<SMT> sh;
  __shared__ float s_lse[16];
  __shared__ uint32_t s_mn[SMT / 64], s_mx[SMT / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int u = blockIdx.x;
  const int G = a.G;
  const int nF = frontier_size(a.v, u);
  frontier_lse<SMT>(a.part, a.W, G, u, s_lse);
  if (tid == 0) sh.lastpos = -1;
  __syncthreads();
  const float invG = 1.0f / (float)G;
  const float* sc = a.scores + (int64_t)u * a.cap1 * G;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for (int pos = tid; pos < nF; pos += SMT) {
    float sv[16];
    load_scores(sc + (int64_t)pos * G, G, true, sv);
    const uint32_t key = mass_key(sv, s_lse, G, invG);
    s_keys[pos] = key;
    mn = min(mn, key);
    mx = max(mx, key);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
  }
  if (lane == 0) { s_mn[wave] = mn; s_mx[wave] = mx; }
  hist_clear(sh);
  __syncthreads();
  uint32_t kmin = s_mn[0], kmax = s_mx[0];
  for (int w = 1; w < SMT / 64; ++w) { kmin = min(kmin, s_mn[w]); kmax = max(kmax, s_mx[w]); }
  uint32_t tau = 0, n_take = 0;
  bool keep_all = a.keep_all || nF == 0;
  if (!keep_all) {
    const u64 span = (u64)kmax - kmin + 1;
    hist_keys<SMT>(sh, s_keys, nF, kmin, span);  // the range covers every key
    __syncthreads();
    if (wave == 0) {
      u64 tot = 0;
      for (int i = lane; i < NB; i += 64) tot += sh.hmass[i];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) tot += __shfl_xor(tot, o);
      if (lane == 0) { sh.T = tot == 0 ? 0 : target_of(a.p, tot); sh.above = 0; }
    }
    __syncthreads();
    const u64 T = sh.T;
    if (T == 0) {
      keep_all = true;  // every mass rounds to zero
    } else {
      tau = refine_cut<SMT>(sh, s_keys, nF, kmin, span, T);
      n_take = ties_to_take(tau, T, sh.above);
    }
  }
  // compaction in position order (chunks of SMT * 4 positions)
  int32_t* kept = a.kept + (int64_t)u * a.capl;
  const int32_t* par = a.v.parent ? a.v.parent + (int64_t)u * a.v.cap_parent : nullptr;
  uint32_t kept_base = 0, tie_base = 0;
  for (int base = 0; base < nF; base += SMT * 4) {
    const int p0 = base + tid * 4;
    uint32_t ngt = 0, neq = 0;
    uint32_t k4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      k4[e] = p0 + e < nF ? s_keys[p0 + e] : 0u;
      if (p0 + e < nF) {
        if (keep_all || k4[e] > tau) ++ngt;
        else if (k4[e] == tau) ++neq;
      }
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan<SMT>((neq << 16) | ngt, &tot, sh.scan);
    const uint32_t avail = n_take > tie_base ? n_take - tie_base : 0;
    const uint32_t taken_before = min(ex >> 16, avail);
    uint32_t take_here = min(neq, avail - taken_before);
    uint32_t out = kept_base + (ex & 0xFFFFu) + taken_before;
    int lastp = -1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (p0 + e < nF) {
        bool keep;
        if (keep_all || k4[e] > tau) keep = true;
        else if (k4[e] == tau && take_here > 0) { keep = true; --take_here; }
        else keep = false;
        if (keep) {
          kept[out++] = frontier_id(par, p0 + e, a.v.C, a.v.Cshift);
          lastp = p0 + e;
        }
      }
    }
    if (lastp >= 0) atomicMax(&sh.lastpos, lastp);
    kept_base += (tot & 0xFFFFu) + min(tot >> 16, avail);
    tie_base += tot >> 16;
    __syncthreads();
  }
  if (tid == 0) {
    a.nF_out[u] = nF;
    a.kept_count[u] = (int)kept_base;
    if (a.next_nF) {
      const int last_id = sh.lastpos >= 0 ? frontier_id(par, sh.lastpos, a.v.C, a.v.Cshift) : 0;
      a.next_nF[u] = next_frontier((int)kept_base, last_id, a.v.C, child_nodes(a.v, u, a.span_child));
    }
  }
}

// --------------------------------------------------------------------------- large levels

struct MassArgs {
  Level v;
  const float* scores;    // [U][cap1][G]
  int64_t cap1;
  const float* part;      // [U][W][G][2] scoring partials
  int W;
  uint32_t* keys;         // [U][kstride]
  int64_t kstride;
  uint32_t* fh_cnt;       // [U][NB] fine histogram (zero on entry; reset by the selection)
  u64* fh_mass;           // [U][NB]
  u64* fh_edge;           // [U][2]: mass above and below the window
  int G, WM;
};

constexpr int MASS_BATCH = 4;

__global__ __launch_bounds__(256) void zha_mass_kernel(MassArgs a) {
  __shared__ float s_lse[16];
  __shared__ uint32_t h_cnt[NB];
  __shared__ u64 h_mass[NB];
  __shared__ u64 s_edge[2][4];
  const int u = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nF = frontier_size(a.v, u);
  const int per = (nF + a.WM - 1) / a.WM;
  const int start = blockIdx.x * per, end = min(nF, start + per);
  if (start >= end) return;
  const int G = a.G;
  frontier_lse<256>(a.part, a.W, G, u, s_lse);
  for (int i = tid; i < NB; i += 256) { h_cnt[i] = 0; h_mass[i] = 0; }
  __syncthreads();
  uint32_t wlo;
  u64 wspan;
  fine_window(nF, &wlo, &wspan);
  const uint32_t whi = (uint32_t)((u64)wlo + wspan - 1);
  const float invG = 1.0f / (float)G;
  const float* sc = a.scores + (int64_t)u * a.cap1 * G;
  uint32_t* keys = a.keys + (int64_t)u * a.kstride;
  u64 am = 0, bm = 0;
  for (int p0 = start + tid; p0 < end; p0 += 256 * MASS_BATCH) {
    float sv[MASS_BATCH][16];
#pragma unroll
    for (int k = 0; k < MASS_BATCH; ++k) {
      const int pos = p0 + 256 * k;
      load_scores(sc + (int64_t)pos * G, G, pos < end, sv[k]);
    }
#pragma unroll
    for (int k = 0; k < MASS_BATCH; ++k) {
      const int pos = p0 + 256 * k;
      if (pos < end) {
        const uint32_t key = mass_key(sv[k], s_lse, G, invG);
        keys[pos] = key;
        if (key > whi) am += fx_mass(key);
        else if (key >= wlo) {
          const uint32_t bn = range_bin(key, wlo, wspan);
          atomicAdd(&h_cnt[bn], 1u);
          atomicAdd(&h_mass[bn], fx_mass(key));
        } else bm += fx_mass(key);
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    am += __shfl_xor(am, o);
    bm += __shfl_xor(bm, o);
  }
  if (lane == 0) { s_edge[0][wave] = am; s_edge[1][wave] = bm; }
  __syncthreads();
  // fold this workgroup's histogram into the unit's (integer atomics: order does not matter)
  uint32_t* gc = a.fh_cnt + (int64_t)u * NB;
  u64* gm = a.fh_mass + (int64_t)u * NB;
  for (int i = tid; i < NB; i += 256)
    if (h_cnt[i]) {
      atomicAdd(&gc[i], h_cnt[i]);
      atomicAdd(&gm[i], h_mass[i]);
    }
  if (tid < 2) {
    const u64 e = s_edge[tid][0] + s_edge[tid][1] + s_edge[tid][2] + s_edge[tid][3];
    if (e) atomicAdd(&a.fh_edge[u * 2 + tid], e);
  }
}

struct LargeArgs {
  Level v;
  const uint32_t* keys;   // [U][kstride]
  int64_t kstride;
  uint32_t* fh_cnt;       // [U][NB]
  u64* fh_mass;
  u64* fh_edge;           // [U][2]
  int32_t* cut;           // [U][4]: tau, last tie position kept, keep_all
  float p;
};

constexpr int LGT = 1024;  // threads of the large-level selection

__device__ __forceinline__ uint4 load4(const uint32_t* k, int pos, int n) {
  if (pos + 3 < n) return *(const uint4*)(k + pos);
  uint4 r = {0u, 0u, 0u, 0u};
  if (pos < n) r.x = k[pos];
  if (pos + 1 < n) r.y = k[pos + 1];
  if (pos + 2 < n) r.z = k[pos + 2];
  return r;
}

// Position of the n-th (0-based) key equal to tau in position order, by counting scans.
__device__ __forceinline__ int nth_tie_scan(SelSh<LGT>& sh, const uint32_t* keys, int nF, uint32_t tau, uint32_t n) {
  uint32_t seen = 0;
  int found = -1;
  for (int base = 0; base < nF && found < 0; base += 4 * LGT) {
    const int p0 = base + 4 * threadIdx.x;
    const uint4 kv = load4(keys, p0, nF);
    const uint32_t k4[4] = {kv.x, kv.y, kv.z, kv.w};
    uint32_t ne = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) ne += (p0 + e < nF && k4[e] == tau) ? 1u : 0u;
    uint32_t tot;
    uint32_t ex = block_excl_scan<LGT>(ne, &tot, sh.scan) + seen;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (p0 + e < nF && k4[e] == tau) {
        if (ex == n) sh.lastpos = p0 + e;
        ++ex;
      }
    __syncthreads();
    seen += tot;
    found = seen > n ? sh.lastpos : -1;
    __syncthreads();
  }
  return found;
}

// Resolves the cut of a large frontier from the fine histogram: the crossing slice's
// keys (with their positions) are gathered into LDS and refined.  A cut outside the
// window, or a slice too full for LDS, falls back to refining over every key.
// Output per unit: tau, and the position of the last tie at tau that is kept (ties are
// taken in position order), so that the compaction is a per-position test.
__global__ __launch_bounds__(LGT) void zha_select_large_kernel(LargeArgs a) {
  __shared__ SelSh<LGT> sh;
  __shared__ u64 s_tot[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int u = blockIdx.x;
  const int nF = frontier_size(a.v, u);
  const uint32_t* keys = a.keys + (int64_t)u * a.kstride;
  uint32_t* gc = a.fh_cnt + (int64_t)u * NB;
  u64* gm = a.fh_mass + (int64_t)u * NB;
  // take the unit's histogram and leave it zeroed for the next level
  for (int i = tid; i < NB; i += LGT) {
    sh.hcnt[i] = gc[i];
    sh.hmass[i] = gm[i];
  }
  if (tid < 2) s_tot[tid] = a.fh_edge[u * 2 + tid];
  __syncthreads();
  for (int i = tid; i < NB; i += LGT) { gc[i] = 0; gm[i] = 0; }
  if (tid < 2) a.fh_edge[u * 2 + tid] = 0;
  uint32_t tau = 0;
  int tie_last = 0x7FFFFFFF;
  int keep_all = nF == 0;
  if (!keep_all) {
    if (wave == 0) {
      u64 wm = 0;
      for (int i = lane; i < NB; i += 64) wm += sh.hmass[i];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) wm += __shfl_xor(wm, o);
      if (lane == 0) {
        const u64 above = s_tot[0], below = s_tot[1], total = above + wm + below;
        const u64 T = total == 0 ? 0 : target_of(a.p, total);
        sh.T = T;
        sh.above = above;
        sh.ncand = (T > above && T <= above + wm) ? 1u : 0u;  // the cut lies in the window
      }
    }
    __syncthreads();
    const u64 T = sh.T;
    if (T == 0) {
      keep_all = 1;  // every mass rounds to zero
    } else {
      uint32_t wlo;
      u64 wspan;
      fine_window(nF, &wlo, &wspan);
      bool gathered = false;
      int nc = 0;
      uint32_t nlo = 0, nhi = 0;
      if (sh.ncand == 1u) {
        if (wave == 0) find_bin(sh.hmass, sh.above, T, &sh.bin, &sh.above);
        __syncthreads();
        slice_range(wlo, wspan, sh.bin, &nlo, &nhi);
        const uint32_t cnt = sh.hcnt[sh.bin];
        __syncthreads();
        if (cnt <= (uint32_t)CAND) {
          if (tid == 0) sh.ncand = 0;
          __syncthreads();
          for (int base = 4 * tid; base < nF; base += 4 * LGT * 2) {
            uint4 kv[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) kv[j] = load4(keys, base + 4 * LGT * j, nF);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const uint32_t ks[4] = {kv[j].x, kv[j].y, kv[j].z, kv[j].w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int pos = base + 4 * LGT * j + e;
                if (pos < nF && ks[e] >= nlo && ks[e] <= nhi) {
                  const uint32_t slot = atomicAdd(&sh.ncand, 1u);
                  sh.ckey[slot] = ks[e];
                  sh.cpos[slot] = (uint32_t)pos;
                }
              }
            }
          }
          __syncthreads();
          nc = (int)sh.ncand;
          gathered = true;
        }
      }
      if (gathered) {
        // refine within the crossing slice over the gathered keys (sh.above: mass above it)
        if (nhi > nlo) {
          const u64 span = (u64)nhi - nlo + 1;
          hist_clear(sh);
          __syncthreads();
          hist_keys<LGT>(sh, sh.ckey, nc, nlo, span);
          __syncthreads();
          tau = refine_cut<LGT>(sh, sh.ckey, nc, nlo, span, T);
        } else {
          tau = nlo;
        }
      } else {
        // general path: every key, over the whole key range
        uint32_t mn = 0xFFFFFFFFu, mx = 0u;
        for (int i = tid; i < nF; i += LGT) { mn = min(mn, keys[i]); mx = max(mx, keys[i]); }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
          mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
          mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
        }
        if (lane == 0) { sh.scan[wave] = mn; sh.red64[wave] = mx; }
        __syncthreads();
        uint32_t kmin = sh.scan[0], kmax = (uint32_t)sh.red64[0];
        for (int w = 1; w < LGT / 64; ++w) { kmin = min(kmin, sh.scan[w]); kmax = max(kmax, (uint32_t)sh.red64[w]); }
        __syncthreads();
        const u64 span = (u64)kmax - kmin + 1;
        hist_clear(sh);
        if (tid == 0) sh.above = 0;
        __syncthreads();
        hist_keys<LGT>(sh, keys, nF, kmin, span);
        __syncthreads();
        tau = refine_cut<LGT>(sh, keys, nF, kmin, span, T);
      }
      const uint32_t n_take = ties_to_take(tau, T, sh.above);
      // ties: the n_take lowest positions among keys equal to tau are kept
      __syncthreads();
      if (tid == 0) sh.neq = 0;
      __syncthreads();
      if (gathered) {
        for (int i = tid; i < nc; i += LGT)
          if (sh.ckey[i] == tau) atomicAdd(&sh.neq, 1u);
        __syncthreads();
        const uint32_t neq = sh.neq;
        if (n_take < neq) {
          // rank each tie by position (ties are rare; only counted when the cut splits them)
          if (tid == 0) sh.lastpos = -1;
          __syncthreads();
          for (int i = tid; i < nc; i += LGT) {
            if (sh.ckey[i] != tau) continue;
            uint32_t rank = 0;
            for (int j = 0; j < nc; ++j) rank += (sh.ckey[j] == tau && sh.cpos[j] < sh.cpos[i]) ? 1u : 0u;
            if (rank == n_take - 1) sh.lastpos = (int)sh.cpos[i];
          }
          __syncthreads();
          tie_last = sh.lastpos;
        }
      } else {
        for (int i = tid; i < nF; i += LGT)
          if (keys[i] == tau) atomicAdd(&sh.neq, 1u);
        __syncthreads();
        if (n_take < sh.neq) tie_last = nth_tie_scan(sh, keys, nF, tau, n_take - 1);
      }
    }
  }
  if (tid == 0) {
    a.cut[u * 4 + 0] = (int32_t)tau;
    a.cut[u * 4 + 1] = tie_last;
    a.cut[u * 4 + 2] = keep_all;
  }
}

struct CompactArgs {
  Level v;
  const uint32_t* keys;   // [U][kstride]
  int64_t kstride;
  const int32_t* cut;     // [U][4]
  int keep_all;           // p >= 1: every position is kept (cut unused)
  u64* status;            // [U][nchunk] look-back words
  int nchunk;
  uint32_t* epoch;        // [2]: epoch of this launch's status words (starts at 1), finished workgroups
  int32_t* last_pos;      // [U] largest kept position (max-reduced; reset by the last chunk)
  int32_t* kept;          // [U][capl]
  int64_t capl;
  int32_t* nF_out;
  int32_t* kept_count;
  int32_t* next_nF;       // null at level 1
  int64_t span_child;
  int32_t* lb_error;      // set when a look-back wait gives up (never expected)
};

constexpr int CPT = 256;  // compaction threads; 4 positions each (CH = 1024 per workgroup)

__device__ __forceinline__ u64 lb_word(uint32_t epoch, int inclusive, uint32_t count) {
  return ((u64)epoch << 32) | ((u64)inclusive << 31) | (u64)count;
}

// Writes the kept ids of one chunk of positions, in order.  Position i is kept when its
// key is above the cut, or equals it and i is not after the last kept tie.  The kept
// counts of earlier chunks arrive by a decoupled look-back over per-chunk status words
// (chunk c waits only on chunks < c, which are dispatched before it).
__device__ __forceinline__ void compact_epilogue(const CompactArgs& a) {
  // the last workgroup of the launch advances the epoch: every workgroup read it before finishing
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t n = gridDim.x * gridDim.y;
    if (atomicAdd(&a.epoch[1], 1u) == n - 1) {
      __hip_atomic_store(&a.epoch[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t e = __hip_atomic_load(&a.epoch[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.epoch[0], e + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

__global__ __launch_bounds__(CPT) void zha_compact_kernel(CompactArgs a) {
  __shared__ uint32_t s_scan[CPT / 64];
  __shared__ uint32_t s_before, s_epoch;
  const int tid = threadIdx.x;
  const int u = blockIdx.y, c = blockIdx.x;
  const int nF = frontier_size(a.v, u);
  const int base = c * CH;
  if (tid == 0) s_epoch = __hip_atomic_load(&a.epoch[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (base >= nF) {
    compact_epilogue(a);
    return;
  }
  const bool keep_all = a.keep_all || a.cut[u * 4 + 2] != 0;
  const uint32_t tau = (uint32_t)a.cut[u * 4 + 0];
  const int tie_last = a.cut[u * 4 + 1];
  const uint32_t* keys = a.keys + (int64_t)u * a.kstride;
  const int p0 = base + 4 * tid;
  uint32_t k4[4] = {0u, 0u, 0u, 0u};
  if (!keep_all) {
    const uint4 kv = load4(keys, p0, nF);
    k4[0] = kv.x; k4[1] = kv.y; k4[2] = kv.z; k4[3] = kv.w;
  }
  bool kp[4];
  uint32_t nk = 0;
  int last_local = -1;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int pos = p0 + e;
    kp[e] = pos < nF && (keep_all || k4[e] > tau || (k4[e] == tau && pos <= tie_last));
    if (kp[e]) { ++nk; last_local = pos; }
  }
  uint32_t tot;
  const uint32_t ex = block_excl_scan<CPT>(nk, &tot, s_scan);
  // largest kept position of the unit, raised (device-scope atomic, completed: its
  // returned value is used below) before this chunk's status word is published
  __shared__ int s_lp[CPT / 64];
  int lp_old = -1;
  if (last_local >= 0) lp_old = atomicMax(&a.last_pos[u], last_local);
  lp_old = max(lp_old, __shfl_xor(lp_old, 32));
  if ((tid & 63) == 0) s_lp[tid >> 6] = lp_old;
  __syncthreads();
  const int lp_seen = max(max(s_lp[0], s_lp[1]), max(s_lp[2], s_lp[3]));
  u64* st = a.status + (int64_t)u * a.nchunk;
  const uint32_t epoch = s_epoch;
  if (tid == 0) {
    uint32_t before = 0;
    const uint32_t dep = lp_seen < -1 ? 1u : 0u;  // always 0: orders the publish after the atomics
    if (c == 0) {
      __hip_atomic_store(&st[0], lb_word(epoch, 1, tot + dep), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      __hip_atomic_store(&st[c], lb_word(epoch, 0, tot + dep), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int i = c - 1; i >= 0; --i) {
        u64 w = 0;
        int spins = 0;
        for (;;) {
          w = __hip_atomic_load(&st[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if ((uint32_t)(w >> 32) == epoch) break;
          if (++spins > (1 << 22)) {  // bounded wait: flag and continue rather than hang
            atomicExch(a.lb_error, 1);
            w = lb_word(epoch, 1, 0);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        before += (uint32_t)(w & 0x7FFFFFFFu);
        if ((w >> 31) & 1) break;
      }
      __hip_atomic_store(&st[c], lb_word(epoch, 1, before + tot), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    s_before = before;
  }
  __syncthreads();
  uint32_t out = s_before + ex;
  int32_t* kept = a.kept + (int64_t)u * a.capl;
  const int32_t* par = a.v.parent ? a.v.parent + (int64_t)u * a.v.cap_parent : nullptr;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (kp[e]) kept[out++] = frontier_id(par, p0 + e, a.v.C, a.v.Cshift);
  // the chunk holding the last position finishes the level's counts: by now every earlier
  // chunk has raised last_pos (before publishing the status words this chunk has read)
  if (base + CH >= nF && tid == 0) {
    const uint32_t total = s_before + tot;
    a.nF_out[u] = nF;
    a.kept_count[u] = (int)total;
    const int lp = __hip_atomic_load(&a.last_pos[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (a.next_nF) {
      const int last_id = lp >= 0 ? frontier_id(par, lp, a.v.C, a.v.Cshift) : 0;
      a.next_nF[u] = next_frontier((int)total, last_id, a.v.C, child_nodes(a.v, u, a.span_child));
    }
    __hip_atomic_store(&a.last_pos[u], -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  compact_epilogue(a);
}

template <typename T, int R, int D>
hipError_t launch_score(const ScoreArgs& a, int W, int U, hipStream_t s) {
  hipLaunchKernelGGL((zha_score_kernel<T, R, D, 2>), dim3(W, U), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_score_r(const ScoreArgs& a, int R, int W, int U, hipStream_t s) {
  switch (R) {
    case 1: return launch_score<T, 1, D>(a, W, U, s);
    case 2: return launch_score<T, 2, D>(a, W, U, s);
    case 4: return launch_score<T, 4, D>(a, W, U, s);
    case 8: return launch_score<T, 8, D>(a, W, U, s);
    default: return launch_score<T, 16, D>(a, W, U, s);
  }
}

int cshift_of(int C) {
  if (C <= 0 || (C & (C - 1)) != 0) return -1;
  int s = 0;
  while ((1 << s) < C) ++s;
  return s;
}

}  // namespace

// Score workgroups per unit at a level: about one 8-node super-tile each at small
// levels, at most t->WS.
int zha_score_wgs(const zha_tree* t, int level) {
  int64_t w = (t->cap[level] + 7) / 8;
  if (w < 1) w = 1;
  if (w > t->WS) w = t->WS;
  return (int)w;
}

int zha_compact_chunks(int64_t nodes) { return (int)((nodes + CH - 1) / CH); }
int zha_hist_bins() { return NB; }

hipError_t zha_launch_route(zha_tree* t, const void* q, float p, float scale, hipStream_t s) {
  const int U = t->U, L = t->L;
  const int Cshift = cshift_of(t->C);
  int32_t* cntF = t->counts;                         // [L+2][U]
  int32_t* cntK = t->counts + (int64_t)(L + 2) * U;  // [L+2][U]
  const bool keep_all = p >= 1.0f;
  hipError_t e;
  for (int l = L; l >= 1; --l) {
    Level v;
    v.parent = l < L ? t->kept[l + 1] : nullptr;
    v.parent_nF = l < L ? cntF + (int64_t)l * U : nullptr;  // written by level l+1
    v.cap_parent = l < L ? t->cap[l + 1] : 0;
    v.span_l = t->span[l];
    v.C = t->C;
    v.Cshift = Cshift;
    v.Hkv = t->desc.n_kv_heads;
    v.len = t->len;
    int32_t* next_nF = l > 1 ? cntF + (int64_t)(l - 1) * U : nullptr;
    const int64_t span_child = l > 1 ? t->span[l - 1] : 1;

    ScoreArgs sa;
    sa.v = v;
    sa.m = t->m[l];
    sa.b = t->b[l];
    sa.q = q;
    sa.capl = t->cap[l];
    sa.scores = t->scores;
    sa.cap1 = t->cap[1];
    sa.part = t->spart;
    sa.W = zha_score_wgs(t, l);
    sa.Hq = t->desc.n_q_heads;
    sa.G = t->G;
    sa.scale = scale;
    zha_time_begin(t, s, ZHA_K_SCORE, l);
    if (t->desc.dtype == ZHA_BF16)
      e = t->d == 64 ? launch_score_r<__bf16, 64>(sa, t->R, sa.W, U, s) : launch_score_r<__bf16, 128>(sa, t->R, sa.W, U, s);
    else
      e = t->d == 64 ? launch_score_r<float, 64>(sa, t->R, sa.W, U, s) : launch_score_r<float, 128>(sa, t->R, sa.W, U, s);
    if (e != hipSuccess) return e;
    zha_time_end(t, s, ZHA_K_SCORE, l);

    if (t->cap[l] <= SMALL_NODES) {
      SmallArgs sm;
      sm.v = v;
      sm.scores = t->scores;
      sm.cap1 = t->cap[1];
      sm.part = t->spart;
      sm.W = sa.W;
      sm.kept = t->kept[l];
      sm.capl = t->cap[l];
      sm.nF_out = cntF + (int64_t)l * U;
      sm.kept_count = cntK + (int64_t)l * U;
      sm.next_nF = next_nF;
      sm.span_child = span_child;
      sm.G = t->G;
      sm.p = p;
      sm.keep_all = keep_all ? 1 : 0;
      zha_time_begin(t, s, ZHA_K_SELECT, l);
      hipLaunchKernelGGL(zha_select_small_kernel, dim3(U), dim3(SMT), 0, s, sm);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      zha_time_end(t, s, ZHA_K_SELECT, l);
      continue;
    }
    if (!keep_all) {
      MassArgs ma;
      ma.v = v;
      ma.scores = t->scores;
      ma.cap1 = t->cap[1];
      ma.part = t->spart;
      ma.W = sa.W;
      ma.keys = t->keys;
      ma.kstride = t->kstride;
      ma.fh_cnt = t->fh_cnt;
      ma.fh_mass = (u64*)t->fh_mass;
      ma.fh_edge = (u64*)t->fh_edge;
      ma.G = t->G;
      int64_t wm = (t->cap[l] + 1023) / 1024;
      ma.WM = (int)(wm > 256 ? 256 : (wm < 1 ? 1 : wm));
      zha_time_begin(t, s, ZHA_K_MASS, l);
      hipLaunchKernelGGL(zha_mass_kernel, dim3(ma.WM, U), dim3(256), 0, s, ma);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      zha_time_end(t, s, ZHA_K_MASS, l);

      LargeArgs la;
      la.v = v;
      la.keys = t->keys;
      la.kstride = t->kstride;
      la.fh_cnt = t->fh_cnt;
      la.fh_mass = (u64*)t->fh_mass;
      la.fh_edge = (u64*)t->fh_edge;
      la.cut = t->cut;
      la.p = p;
      zha_time_begin(t, s, ZHA_K_SELECT, l);
      hipLaunchKernelGGL(zha_select_large_kernel, dim3(U), dim3(LGT), 0, s, la);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      zha_time_end(t, s, ZHA_K_SELECT, l);
    }
    CompactArgs ca;
    ca.v = v;
    ca.keys = t->keys;
    ca.kstride = t->kstride;
    ca.cut = t->cut;
    ca.keep_all = keep_all ? 1 : 0;
    ca.status = (u64*)t->lb_status;
    ca.nchunk = zha_compact_chunks(t->cap[1]);
    ca.epoch = t->lb_epoch;  // device-side: graph replays keep advancing it
    ca.last_pos = t->last_pos;
    ca.kept = t->kept[l];
    ca.capl = t->cap[l];
    ca.nF_out = cntF + (int64_t)l * U;
    ca.kept_count = cntK + (int64_t)l * U;
    ca.next_nF = next_nF;
    ca.span_child = span_child;
    ca.lb_error = t->lb_error;
    const int nch = zha_compact_chunks(t->cap[l]);
    zha_time_begin(t, s, ZHA_K_COMPACT, l);
    hipLaunchKernelGGL(zha_compact_kernel, dim3(nch, U), dim3(CPT), 0, s, ca);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    zha_time_end(t, s, ZHA_K_COMPACT, l);
  }
  return hipSuccess;
}
