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
// Per level two kernels run:
//   zha_score_kernel   many workgroups per unit; streams the frontier's planes from
//                      HBM once and scores them on the matrix cores (the G query
//                      heads times the R planes of a node is a small dense product);
//                      writes the scores and per-workgroup log-sum-exp partials.
//   zha_select_kernel  one 1024-thread workgroup per unit; normalises, forms the
//                      node masses, finds the exact top-p cut by radix selection on
//                      the fp32 mass bits with fixed-point (integer) mass sums, and
//                      compacts the kept ids in ascending order.
// Integer sums make the selection independent of summation order, so results
// are bit-identical from run to run.
#include "zha_internal.h"

namespace {

struct ScoreArgs {
  const void* m;          // level planes m [U][capl][R][d]
  const float* b;         // level planes b [U][capl][R]
  const void* q;          // [B][Hq][d]
  const int32_t* parent;  // kept ids of level l+1 [U][cap_parent]; null at the top level
  int64_t cap_parent;
  int64_t capl;
  const int32_t* nF;      // frontier counts of this level [U]; null at the top level
  float* scores;          // [U][cap1][G]
  int64_t cap1;
  float* part;            // [U][W][G][2] (max, sum exp) of the workgroup's scores per head
  int W;                  // workgroups per unit
  int Hkv, Hq, G, C, Cshift;
  int64_t span_l;         // tokens per node at this level, C^l
  float scale;
  ZLens len;
};

__device__ __forceinline__ int frontier_size(const int32_t* nF, int u, int bi, const ZLens& len, int C,
                                             int64_t span) {
  if (nF) return nF[u];
  int64_t N = len.n[bi];
  int64_t Nc = (N / C) * C;
  return (int)((Nc + span - 1) / span);
}

// Node id of frontier position pos: the top level lists every node; a lower level
// lists the children of the kept parents in order (only the last parent can be partial).
__device__ __forceinline__ int frontier_id(const int32_t* parent, int pos, int C, int Cshift) {
  if (!parent) return pos;
  if (Cshift >= 0) return (parent[pos >> Cshift] << Cshift) + (pos & ((1 << Cshift) - 1));
  int k = pos / C;
  return parent[k] * C + (pos - k * C);
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
  float mx = fmaxf(M, M2);
  if (mx == -INFINITY) { M = -INFINITY; S = 0.0f; return; }
  S = S * zexp(M - mx) + S2 * zexp(M2 - mx);
  M = mx;
}

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
  const int u = blockIdx.y, bi = u / a.Hkv, g = u % a.Hkv;
  const int G = a.G;
  const int nF = frontier_size(a.nF, u, bi, a.len, a.C, a.span_l);
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
  const int32_t* par = a.parent ? a.parent + (int64_t)u * a.cap_parent : nullptr;
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
      const int id = v ? frontier_id(par, pos, a.C, a.Cshift) : 0;
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
    M2 = __shfl_xor(runM, 32); S2 = __shfl_xor(runS, 32);
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

// --------------------------------------------------------------------------------- select

struct SelectArgs {
  const float* scores;    // [U][cap1][G]
  int64_t cap1;
  const float* part;      // [U][W][G][2]
  int W;
  uint32_t* keys;         // [U][cap1] scratch
  const int32_t* nF;      // frontier counts [U]; null at the top level
  int32_t* nF_out;        // frontier counts of this level, written for inspection [U]
  const int32_t* parent;  // kept ids of level l+1 [U][cap_parent]; null at the top level
  int64_t cap_parent;
  int32_t* kept;          // kept ids of this level [U][capl]
  int64_t capl;
  int32_t* kept_count;    // [U]
  int32_t* next_nF;       // frontier counts of level l-1 [U]; null at level 1
  int G, C, Cshift, Hkv;
  int64_t span_l, span_child;
  float p;
  int keep_all;
  ZLens len;
};

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int SEL_PER = 16;  // positions per thread per compaction chunk

typedef unsigned long long u64;

// Fixed-point mass: w * 2^40 truncated (w <= 1 up to rounding).  Exact integer sums
// make every cumulative mass independent of the order of summation.
__device__ __forceinline__ u64 fx_mass(uint32_t key) {
  return (u64)(__uint_as_float(key) * 1099511627776.0f);
}

// Exclusive scan of one u32 per thread over the workgroup; returns the total in *tot.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* tot, uint32_t* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    uint32_t v = lane < SEL_WAVES ? sh[lane] : 0u;
    uint32_t vi = v;
#pragma unroll
    for (int o = 1; o < SEL_WAVES; o <<= 1) {
      uint32_t y = __shfl_up(vi, o);
      if (lane >= o) vi += y;
    }
    if (lane < SEL_WAVES) sh[SEL_WAVES + lane] = vi - v;
    if (lane == SEL_WAVES - 1) sh[2 * SEL_WAVES] = vi;
  }
  __syncthreads();
  uint32_t r = sh[SEL_WAVES + wave] + inc - x;
  *tot = sh[2 * SEL_WAVES];
  __syncthreads();
  return r;
}

// Given a 256-bin histogram (count, fixed-point mass) and the mass already above the
// bins, find the bin in which the cumulative mass, from the heaviest bin down,
// reaches T.  Wave 0 only; results to *bin, *above, *cabove.
__device__ __forceinline__ void find_bin(const uint32_t* hc, const u64* hm, u64 above0, uint32_t cabove0, u64 T,
                                         uint32_t* out_bin, u64* out_above, uint32_t* out_cabove) {
  const int lane = threadIdx.x & 63;
  // lane l owns bins 255-4l ... 252-4l (heaviest first)
  u64 m4[4];
  uint32_t c4[4];
  u64 ls = 0;
  uint32_t lc = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int bin = 255 - 4 * lane - e;
    m4[e] = hm[bin];
    c4[e] = hc[bin];
    ls += m4[e];
    lc += c4[e];
  }
  u64 inc = ls;
  uint32_t cinc = lc;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    u64 y = __shfl_up(inc, o);
    uint32_t cy = __shfl_up(cinc, o);
    if (lane >= o) { inc += y; cinc += cy; }
  }
  u64 run = above0 + inc - ls;
  uint32_t crun = cabove0 + cinc - lc;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (run < T && run + m4[e] >= T) {
      *out_bin = 255 - 4 * lane - e;
      *out_above = run;
      *out_cabove = crun;
    }
    run += m4[e];
    crun += c4[e];
  }
}

__global__ __launch_bounds__(SEL_THREADS) void zha_select_kernel(SelectArgs a) {
  __shared__ float s_lse[16];
  __shared__ uint32_t h_cnt[256];
  __shared__ u64 h_mass[256];
  __shared__ uint32_t s_scan[2 * SEL_WAVES + 1];
  __shared__ uint32_t s_prefix, s_cabove, s_bin;
  __shared__ u64 s_above, s_T;
  __shared__ int s_last_id;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int u = blockIdx.x, bi = u / a.Hkv;
  const int G = a.G;
  const int64_t N = a.len.n[bi];
  const int64_t Nc = (N / a.C) * a.C;
  const int nF = frontier_size(a.nF, u, bi, a.len, a.C, a.span_l);
  const int n_child = (int)((Nc + a.span_child - 1) / a.span_child);
  if (tid == 0) a.nF_out[u] = nF;
  if (nF == 0) {
    if (tid == 0) {
      a.kept_count[u] = 0;
      if (a.next_nF) a.next_nF[u] = 0;
    }
    return;
  }
  // per-head log-sum-exp over the frontier from the scoring workgroups' partials
  if (wave < G) {
    float Mx = -INFINITY, Sx = 0.0f;
    for (int i = lane; i < a.W; i += 64) {
      const float* pp = a.part + (((int64_t)u * a.W + i) * G + wave) * 2;
      lse_merge(Mx, Sx, pp[0], pp[1]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      float M2 = __shfl_xor(Mx, o), S2 = __shfl_xor(Sx, o);
      lse_merge(Mx, Sx, M2, S2);
    }
    if (lane == 0) s_lse[wave] = Mx + zlog(Sx);
  }
  if (tid < 256) { h_cnt[tid] = 0; h_mass[tid] = 0; }
  __syncthreads();
  const float invG = 1.0f / (float)G;
  uint32_t* keys = a.keys + (int64_t)u * a.cap1;
  const float* sc = a.scores + (int64_t)u * a.cap1 * G;
  // node masses w = mean over heads of exp(s - lse); key = fp32 bits of w (monotone in w)
  for (int pos = tid; pos < nF; pos += SEL_THREADS) {
    const float* sp = sc + (int64_t)pos * G;
    float w = 0.0f;
    for (int h = 0; h < G; ++h) w += zexp(sp[h] - s_lse[h]);
    w *= invG;
    const uint32_t key = __float_as_uint(w);
    keys[pos] = key;
    if (!a.keep_all) {
      atomicAdd(&h_cnt[key >> 24], 1u);
      atomicAdd(&h_mass[key >> 24], fx_mass(key));
    }
  }
  __syncthreads();
  uint32_t tau = 0;
  u64 n_take = 0;
  int keep_all = a.keep_all;
  if (!keep_all) {
    // total mass and target p * W (integer, rounded up: c >= p*W <=> c >= ceil(p*W))
    if (wave == 0) {
      u64 s = 0;
      for (int i = lane; i < 256; i += 64) s += h_mass[i];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
      if (lane == 0) {
        double tgt = ceil((double)a.p * (double)s);
        u64 T = (u64)tgt;
        if (T < 1) T = 1;
        if (T > s) T = s;
        s_T = T;  // 0 only when every mass rounds to zero: keep everything
      }
    }
    __syncthreads();
    if (s_T == 0) keep_all = 1;
  }
  if (!keep_all) {
    const u64 T = s_T;
    if (wave == 0) find_bin(h_cnt, h_mass, 0, 0, T, &s_bin, &s_above, &s_cabove);
    __syncthreads();
    uint32_t prefix = s_bin;
    for (int d = 1; d < 4; ++d) {
      const int shift_hi = 32 - 8 * d, shift = 24 - 8 * d;
      if (tid < 256) { h_cnt[tid] = 0; h_mass[tid] = 0; }
      __syncthreads();
      for (int pos = tid; pos < nF; pos += SEL_THREADS) {
        const uint32_t key = keys[pos];
        if ((key >> shift_hi) == prefix) {
          const uint32_t dg = (key >> shift) & 255u;
          atomicAdd(&h_cnt[dg], 1u);
          atomicAdd(&h_mass[dg], fx_mass(key));
        }
      }
      __syncthreads();
      if (wave == 0) find_bin(h_cnt, h_mass, s_above, s_cabove, T, &s_bin, &s_above, &s_cabove);
      __syncthreads();
      prefix = (prefix << 8) | s_bin;
    }
    tau = prefix;
    // ties at the cut all carry the same mass; take the fewest that reach T, lowest positions first
    const u64 mt = fx_mass(tau) > 0 ? fx_mass(tau) : 1;  // the cut element always carries mass
    n_take = (T - s_above + mt - 1) / mt;
  }
  // compaction: positions in order, keep = key > tau, or key == tau among the first n_take ties
  int32_t* kept = a.kept + (int64_t)u * a.capl;
  const int32_t* par = a.parent ? a.parent + (int64_t)u * a.cap_parent : nullptr;
  u64 tie_base = 0;
  uint32_t kept_base = 0;
  for (int base = 0; base < nF; base += SEL_THREADS * SEL_PER) {
    const int p0 = base + tid * SEL_PER;
    uint32_t k16[SEL_PER];
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int e = 0; e < SEL_PER; ++e) {
      const int pos = p0 + e;
      k16[e] = pos < nF ? keys[pos] : 0u;
      if (pos < nF) {
        if (keep_all || k16[e] > tau) ++ngt;
        else if (k16[e] == tau) ++neq;
      }
    }
    uint32_t tot;
    const uint32_t packed_excl = block_excl_scan((neq << 16) | ngt, &tot, s_scan);
    const uint32_t gt_excl = packed_excl & 0xFFFFu, eq_excl = packed_excl >> 16;
    const uint32_t gt_tot = tot & 0xFFFFu, eq_tot = tot >> 16;
    // ties taken before this thread and by this thread
    const u64 avail = n_take > tie_base ? n_take - tie_base : 0;
    const uint32_t taken_before = (uint32_t)min((u64)eq_excl, avail);
    uint32_t taken_here = (uint32_t)min((u64)neq, avail - taken_before);
    uint32_t out = kept_base + gt_excl + taken_before;
    uint32_t eq_seen = 0;
#pragma unroll
    for (int e = 0; e < SEL_PER; ++e) {
      const int pos = p0 + e;
      if (pos >= nF) break;
      bool keep;
      if (keep_all || k16[e] > tau) keep = true;
      else if (k16[e] == tau) { keep = eq_seen < taken_here; ++eq_seen; }
      else keep = false;
      if (keep) {
        const int id = frontier_id(par, pos, a.C, a.Cshift);
        kept[out] = id;
        ++out;
      }
    }
    const uint32_t taken_tot = (uint32_t)min((u64)eq_tot, avail);
    kept_base += gt_tot + taken_tot;
    tie_base += eq_tot;
    (void)taken_here;
  }
  __syncthreads();
  if (tid == 0) {
    a.kept_count[u] = (int)kept_base;
    if (a.next_nF) {
      if (kept_base == 0) {
        a.next_nF[u] = 0;
      } else {
        const int last = kept[kept_base - 1];
        const int nlast = min(a.C, n_child - last * a.C);
        a.next_nF[u] = a.C * (int)(kept_base - 1) + nlast;
      }
    }
  }
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

}  // namespace

int zha_score_wgs(const zha_tree* t, int level) {
  // about 16 nodes per workgroup at least, at most t->WS workgroups per unit
  int64_t w = (t->cap[level] + 15) / 16;
  if (w < 1) w = 1;
  if (w > t->WS) w = t->WS;
  return (int)w;
}

hipError_t zha_launch_route(zha_tree* t, const void* q, float p, float scale, hipStream_t s) {
  const int U = t->U, L = t->L;
  int Cshift = -1;
  if ((t->C & (t->C - 1)) == 0) { Cshift = 0; while ((1 << Cshift) < t->C) ++Cshift; }
  int32_t* cntF = t->counts;                       // [L+2][U]
  int32_t* cntK = t->counts + (int64_t)(L + 2) * U;  // [L+2][U]
  for (int l = L; l >= 1; --l) {
    ScoreArgs sa;
    sa.m = t->m[l];
    sa.b = t->b[l];
    sa.q = q;
    sa.parent = l < L ? t->kept[l + 1] : nullptr;
    sa.cap_parent = l < L ? t->cap[l + 1] : 0;
    sa.capl = t->cap[l];
    sa.nF = l < L ? cntF + (int64_t)l * U : nullptr;
    sa.scores = t->scores;
    sa.cap1 = t->cap[1];
    sa.part = t->spart;
    sa.W = zha_score_wgs(t, l);
    sa.Hkv = t->desc.n_kv_heads;
    sa.Hq = t->desc.n_q_heads;
    sa.G = t->G;
    sa.C = t->C;
    sa.Cshift = Cshift;
    sa.span_l = t->span[l];
    sa.scale = scale;
    sa.len = t->len;
    zha_time_begin(t, s);
    hipError_t e;
    if (t->desc.dtype == ZHA_BF16)
      e = t->d == 64 ? launch_score_r<__bf16, 64>(sa, t->R, sa.W, U, s) : launch_score_r<__bf16, 128>(sa, t->R, sa.W, U, s);
    else
      e = t->d == 64 ? launch_score_r<float, 64>(sa, t->R, sa.W, U, s) : launch_score_r<float, 128>(sa, t->R, sa.W, U, s);
    if (e != hipSuccess) return e;
    zha_time_end(t, s, ZHA_K_SCORE, l);

    SelectArgs se;
    se.scores = t->scores;
    se.cap1 = t->cap[1];
    se.part = t->spart;
    se.W = sa.W;
    se.keys = t->keys;
    se.nF = sa.nF;
    se.nF_out = cntF + (int64_t)l * U;
    se.parent = sa.parent;
    se.cap_parent = sa.cap_parent;
    se.kept = t->kept[l];
    se.capl = t->cap[l];
    se.kept_count = cntK + (int64_t)l * U;
    se.next_nF = l > 1 ? cntF + (int64_t)(l - 1) * U : nullptr;
    se.G = t->G;
    se.C = t->C;
    se.Cshift = Cshift;
    se.Hkv = t->desc.n_kv_heads;
    se.span_l = t->span[l];
    se.span_child = l > 1 ? t->span[l - 1] : 1;
    se.p = p;
    se.keep_all = p >= 1.0f ? 1 : 0;
    se.len = t->len;
    zha_time_begin(t, s);
    hipLaunchKernelGGL(zha_select_kernel, dim3(U), dim3(SEL_THREADS), 0, s, se);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    zha_time_end(t, s, ZHA_K_SELECT, l);
  }
  return hipSuccess;
}
