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
//   levels of <= 1024 nodes: selected by the next level's scoring launch, every one of
//                       whose workgroups first repeats the selection (a 256-thread block:
//                       LSE per head, keys, a histogram, the crossing bin ranked by one
//                       wave, ordered compaction) from the scores, then scores its share of
//                       the frontier that selection defines; level 1 of that size takes
//                       zha_select_wave_kernel, the same selection in its own launch.
//   levels of <= 8192 nodes: zha_select_small_kernel, one workgroup per unit,
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
#include <algorithm>

#include "zha_internal.h"

namespace {

constexpr int NB = 1024;                 // histogram slices
constexpr int SMALL_NODES = 8192;        // frontiers up to this size are selected in one workgroup
constexpr int CH = 4096;                 // compaction chunk (positions per workgroup)

// Per-level inputs shared by the kernels of one level.  Node counts per sequence come from
// the tree's geometry table (written by the build and append kernels), so the launch
// arguments stay small (a launch's cost grows with the size of its arguments).
struct Level {
  const int32_t* parent;      // kept ids of level l+1 [U][cap_parent]; null at the top level
  const int32_t* parent_nF;   // frontier counts of this level, written by level l+1 [U]
  int64_t cap_parent;
  int C, Cshift, Hkv;
  const int32_t* nodes;       // nodes of this level per sequence [B]
  const int32_t* child;       // nodes of level l-1 per sequence [B] (unused at level 1)
};

__device__ __forceinline__ int frontier_size(const Level& v, int u) {
  if (v.parent) return v.parent_nF[u];
  return v.nodes[u / v.Hkv];
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

__device__ __forceinline__ int child_nodes(const Level& v, int u) { return v.child[u / v.Hkv]; }

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

// Fixed-point mass of a key: w * 2^40 truncated (w <= 1 up to rounding), from the bits:
// w = m * 2^(e - 150) with m the 24-bit significand, so w * 2^40 = m * 2^(e - 110).
// Branch-free; zero and subnormal keys (far below the 2^-40 resolution) give 0.
__device__ __forceinline__ u64 fx_mass(uint32_t key) {
  const int e = (int)(key >> 23) & 0xFF;
  const u64 m = (u64)((key & 0x7FFFFFu) | 0x800000u);
  const int sft = e - 110;
  const u64 up = m << min(max(sft, 0), 63);
  const u64 dn = m >> min(max(-sft, 0), 63);
  const u64 r = sft >= 0 ? up : dn;
  return e == 0 ? 0 : r;
}

// Score rows hold the G heads' scores of one node padded to a multiple of 4 floats
// (16-byte aligned rows; the padding is never read as a score).
__device__ __forceinline__ int score_stride(int G) { return (G + 3) & ~3; }

// Node mass key from its G scores: mean over heads of exp(s_h - LSE_h), as fp32 bits.
__device__ __forceinline__ uint32_t mass_key(const float4 (&sv)[4], const float* lse, int G, float invG) {
  float w = 0.0f;
#pragma unroll
  for (int h4 = 0; h4 < 4; ++h4) {
    if (4 * h4 < G) {
      const float4 v = sv[h4];
      w += zexp(v.x - lse[4 * h4]);
      w += 4 * h4 + 1 < G ? zexp(v.y - lse[4 * h4 + 1]) : 0.0f;
      w += 4 * h4 + 2 < G ? zexp(v.z - lse[4 * h4 + 2]) : 0.0f;
      w += 4 * h4 + 3 < G ? zexp(v.w - lse[4 * h4 + 3]) : 0.0f;
    }
  }
  return __float_as_uint(w * invG);
}

// The scores of one node (sp must point at a readable row: callers clamp the position;
// the head bound is uniform, so only whole float4 groups are skipped).
__device__ __forceinline__ void load_scores(const float* sp, int G, float4 (&sv)[4]) {
#pragma unroll
  for (int h4 = 0; h4 < 4; ++h4)
    sv[h4] = 4 * h4 < G ? *(const float4*)(sp + 4 * h4) : make_float4(0.f, 0.f, 0.f, 0.f);
}

// ----------------------------------------------------------------------------------- score

struct ScoreArgs {
  Level v;
  const void* m;          // level planes m [U][capl][R][d] (tree dtype, or fp8 e4m3 codes)
  const float* b;         // level planes b [U][capl][R]
  const float* ms;        // fp8 summaries: row scales [U][capl][R]
  const void* q;          // [B][Tq][Hq][d]
  int64_t capl;
  float* scores;          // [U][cap1][G]
  int64_t cap1;
  float* part;            // [U][W][G][2]: (max, sum exp) of the workgroup's scores per head
  int W;                  // workgroups per unit (per group of units when scoring unions)
  int G;                  // query heads per routing unit
  int hr;                 // routing units per (query, KV head): 1, or Gq when each head is routed alone
  int Hkv, Tq;            // KV heads; queries per sequence
  float scale;
  // Union scoring: one row of workgroups per group of the routing units that share one
  // (sequence, KV head): the hr units of each of TS consecutive queries (TS * Gq <= 16
  // matrix columns).  A node is scored once for every column; a unit keeps the scores of
  // the nodes of its own frontier.
  const u64* krank;       // [RU][cap_parent]: the parent level's kept nodes, (stamp << 32) | rank in
                          // the unit's kept list; null at the top level (every node is a member)
  uint32_t* route_ctr;    // route stamp; the top level's first workgroup advances it
  int TS, NTC;            // queries per group; groups per (sequence, KV head)
  // PSEL (one routing unit per grid row): the parent level l+1 has at most WN frontier nodes
  // and was scored but not selected; every workgroup selects it itself (one wave, from the
  // parent level's scores and partials) and scores the children of its kept nodes.
  // Workgroup 0 of each unit publishes the parent level's selection.
  Level pv;               // the parent level (its frontier: pv.parent, pv.parent_nF, pv.nodes)
  const float* pscores;   // the parent level's scores [U][pstride][score row]
  int64_t pstride;
  int32_t* pkept;         // kept ids of the parent level [U][pcapl] (written by workgroup 0)
  int64_t pcapl;
  int32_t* pnF_out;       // the parent level's frontier counts [U]
  int32_t* pkept_count;   // the parent level's kept counts [U]
  int32_t* nF_out;        // this level's frontier counts [U]
  float p;
  int keep_all;
};

// Selection of a level of at most WN frontier nodes by one wave (see wave_select).
constexpr int WN = 1024;
struct WaveSh {
  uint32_t keys[WN];      // mass keys by frontier position
  int32_t fid[WN];        // node ids by frontier position
  int32_t kept[WN];       // kept node ids, ascending
  uint32_t hcnt[1024];    // histogram of the key range
  u64 hmass[1024];
  uint32_t ckey[64], cpos[64];
};
__device__ void wave_select(const Level& v, int u, int capF, const float* scores, int64_t sstride, int G, float p,
                            int keep_all, WaveSh& sh, int& nF_out, int& nk_out, int& nx_out);

// Eight fp8 e4m3 codes (two dwords) as eight bf16 values (exact), by the hardware
// conversion; element e is byte e.
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 r;
  const uint32_t w[2] = {lo, hi};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const auto f01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
    const auto f23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
    // upper halves of the floats: bf16 values, exact (an e4m3 value has 4 significant bits)
    r[2 * i] = __builtin_amdgcn_perm(__float_as_uint(f01[1]), __float_as_uint(f01[0]), 0x07060302u);
    r[2 * i + 1] = __builtin_amdgcn_perm(__float_as_uint(f23[1]), __float_as_uint(f23[0]), 0x07060302u);
  }
  return __builtin_bit_cast(bf16x8_t, r);
}

// Eight fp4 e2m1 codes (one dword, element 2i in the low nibble of byte i) as eight bf16
// values times the block scale sc (exact: two significant bits and a power of two).
__device__ __forceinline__ bf16x8_t fp4x8_to_bf16(uint32_t w, float sc) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3);
  bf16x8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Scores one level's frontier.  Rows of an MFMA tile are (node, reference query)
// pairs: 16/R nodes per tile; columns are the KV head's query heads (G <= 16).
// Lane i loads its row's plane slice (k-slot group i/16) straight from HBM; the
// query fragments stay in registers for the whole workgroup.  F8: the planes are fp8
// codes; lane (row, group) loads its row's d/4 contiguous codes, decodes them to bf16 in
// registers, and the query fragments take the same k order (the dot product does not
// depend on it); the row's scale multiplies the product.  F4 (SM = 2): the lane's d/4 values
// are one block-of-32's share (d = 128: the whole block), decoded with the block scale.
// UNI (R >= 4): the workgroup row scores the union of the frontiers of a group of routing
// units in node-id order, in NT column tiles of 16 (column c = 16 * tile + lane row is head
// jcol of unit cu(c)): every loaded plane tile feeds NT matrix products.  A node is loaded
// when some column's unit has its parent kept (a stamped rank entry), and each column keeps
// the scores of its unit's member nodes at the unit's frontier positions.
// PO2: the chunk is a power of two, so node and parent ids are shifts (the generic form divides
// by C under a branch on every id).
template <typename T, int R, int D, int UN, int SM, bool UNI, int NT, bool PSEL, bool PO2 = false>
__global__ __launch_bounds__(256, UNI ? 2 : (PSEL ? 3 : 4)) void zha_score_kernel(ScoreArgs a) {
  typedef Mf<T> M;
  static_assert(!PSEL || !UNI, "in-kernel parent selection serves one routing unit per grid row");
  constexpr bool F8 = SM == 1, F4 = SM == 2, LP = SM != 0;  // summary storage: native, fp8, fp4
  // FLAT: loads are issued unconditionally (inactive rows read a clamped, readable address and
  // their results are discarded), so no load sits under a branch, after whose join the compiler
  // waits for every load in flight.  Taken where it measured faster (union scoring, fp4 planes);
  // the bandwidth-bound native and fp8 per-unit kernels keep guarded loads, which spare the
  // small levels the reads of rows past the frontier.
  constexpr bool FLAT = UNI || F4;
  constexpr int NK = D / M::KPER;
  constexpr int NR = F8 ? D / 64 : 1;   // 16-byte code loads per lane per tile (F8; F4 uses one)
  constexpr int NPT = 16 / R;
  constexpr int SUPER = 4 * UN * NPT;
  static_assert(!LP || M::EPL == 8, "fp8 and fp4 planes feed the bf16 matrix instruction");
  static_assert(!F4 || D % 64 == 0, "fp4 lanes hold whole code words");
  static_assert(!UNI || R >= 4, "union scoring keeps one node per lane group");
  static_assert(UNI || NT == 1, "one column tile unless scoring unions");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool csh = PO2 || a.v.Cshift >= 0;
  const int row = lane & 15, grp = lane >> 4;
  const int G = a.G;
  // per column tile n: u[n] the routing unit (frontier, scores, partials) of this lane's
  // column, jc[n] its head in the unit, ok[n] the column is a query head; up: the (sequence,
  // KV head) unit whose planes are scored
  int u[NT], jc[NT], up, end;
  bool ok[NT];
  if constexpr (UNI) {
    up = blockIdx.y / a.NTC;
    const int tc = blockIdx.y - up * a.NTC, bi = up / a.Hkv, g = up - bi * a.Hkv;
    const int per_t = a.hr * G;  // columns per query
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int col = 16 * n + row;
      const int tt = col / per_t, h = (col / G) % a.hr, t = tc * a.TS + tt;
      ok[n] = tt < a.TS && t < a.Tq;
      u[n] = ((bi * a.Tq + min(t, a.Tq - 1)) * a.Hkv + g) * a.hr + h;
      jc[n] = col % G;
    }
    end = a.v.nodes[bi];
    if (a.route_ctr && !a.krank && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
      // top level of a route: a new stamp, so kept ranks written by earlier routes stop matching
      const uint32_t s0 = __hip_atomic_load(a.route_ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.route_ctr, s0 + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else {
    u[0] = blockIdx.y;
    up = plane_unit(u[0], a.hr, a.Hkv, a.Tq);
    ok[0] = row < G;
    jc[0] = row;
    end = PSEL ? 0 : frontier_size(a.v, u[0]);
  }
  const uint32_t stamp = (UNI && a.krank) ? a.route_ctr[0] : 0u;
  // Super-tiles are dealt to the workgroups in turn: at any moment the unit's workgroups
  // read neighbouring addresses, sweeping the planes in order.
  const int start = blockIdx.x * SUPER;
  const int step = a.W * SUPER;

  // PSEL: the workgroup selects the parent level first (its query loads then go out with
  // the first plane loads); the kept parents are read from LDS
  __shared__ WaveSh wsh_[1];  // referenced by the PSEL instantiations only
  if constexpr (PSEL) {
    WaveSh& wsh = wsh_[0];
    int nFp, nk, nx;
    wave_select(a.pv, u[0], (int)a.pcapl, a.pscores, a.pstride, G, a.p, a.keep_all, wsh, nFp, nk, nx);
    end = nx;
    if (blockIdx.x == 0) {  // publish the parent level's selection (one workgroup per unit)
      if (threadIdx.x == 0) {
        a.pnF_out[u[0]] = nFp;
        a.pkept_count[u[0]] = nk;
        a.nF_out[u[0]] = nx;
      }
      int32_t* kp = a.pkept + (int64_t)u[0] * a.pcapl;
      for (int i = threadIdx.x; i < nk; i += blockDim.x) kp[i] = wsh.kept[i];
    }
  }
  typename M::frag qf[NT][NK];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const T* qp = (const T*)a.q + ((int64_t)u[n] * G + jc[n]) * D;
#pragma unroll
    for (int s = 0; s < NK; ++s) {
      const int k0 = LP ? grp * (D / 4) + s * 8 : s * M::KPER + grp * M::EPL;
      qf[n][s] = ok[n] ? M::load(qp + k0) : M::zero();
    }
  }
  const int32_t* par = (!UNI && !PSEL && a.v.parent) ? a.v.parent + (int64_t)u[0] * a.v.cap_parent : nullptr;
  const bool has_par = PSEL || par != nullptr;
  // always-readable bases for the unconditional parent-id and kept-rank loads (entry 0 is read
  // when the real array is absent or the entry is not needed)
  const int32_t* pload = par ? par : a.v.nodes;
  const u64* kload = a.krank ? a.krank : (const u64*)a.scores;
  const T* mb = (const T*)a.m + (int64_t)up * a.capl * R * D;
  const uint8_t* m8 = (const uint8_t*)a.m + (int64_t)up * a.capl * R * (F4 ? D / 2 : D);
  const float* bb = a.b + (int64_t)up * a.capl * R;
  const float* sb = F8 ? a.ms + (int64_t)up * a.capl * R : nullptr;
  const uint8_t* sb4 = F4 ? (const uint8_t*)a.ms + (int64_t)up * a.capl * R * (D / 32) : nullptr;
  const int GS = score_stride(G);
  float runM[NT], runS[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) { runM[n] = -INFINITY; runS[n] = 0.0f; }

  typedef typename M::frag Frag;
  // Parent entries of this lane's tiles in the super-tile at `base` (the one load a node
  // id depends on).  UNI: the kept-rank entries of the parent of the lane's node (4grp/R)
  // for the lane's column units.
  auto fetch_par = [&](int base, int (&pp)[UN], u64 (&rk)[UN][NT]) {
#pragma unroll
    for (int k = 0; k < UN; ++k) {
      if constexpr (UNI) {
        const int id = base + (k * 4 + wave) * NPT + (4 * grp) / R;
        const int P = csh ? (id >> a.v.Cshift) : id / a.v.C;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const bool need = a.krank && ok[n] && id < end;
          const u64 x = kload[need ? (int64_t)u[n] * a.v.cap_parent + P : 0];
          rk[k][n] = need ? x : 0;
        }
        pp[k] = 0;
      } else {
        const int pos = base + (k * 4 + wave) * NPT + row / R;
        const bool need = has_par && pos < end;
        const int pidx = need ? (csh ? (pos >> a.v.Cshift) : pos / a.v.C) : 0;
        int32_t x;
        if constexpr (PSEL) x = wsh_[0].kept[pidx];
        else x = (FLAT || need) ? pload[pidx] : 0;
        pp[k] = need ? x : 0;
        rk[k][0] = 0;
      }
    }
  };
  // UNI: membership of the lane's node for its columns (mem), the node's position in each
  // column unit's frontier (wpos), and which nodes of each tile some column needs (act).
  auto members = [&](int base, const u64 (&rk)[UN][NT], bool (&mem)[UN][NT], int (&wpos)[UN][NT],
                     uint32_t (&act)[UN]) {
#pragma unroll
    for (int k = 0; k < UN; ++k) {
      const int id = base + (k * 4 + wave) * NPT + (4 * grp) / R;
      bool any = false;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        bool m;
        int pos;
        if (a.krank) {
          m = ok[n] && id < end && (uint32_t)(rk[k][n] >> 32) == stamp;
          const int rank = (int)(uint32_t)rk[k][n];
          pos = csh ? (rank << a.v.Cshift) + (id & ((1 << a.v.Cshift) - 1)) : rank * a.v.C + id % a.v.C;
        } else {
          m = ok[n] && id < end;
          pos = id;
        }
        mem[k][n] = m;
        wpos[k][n] = pos;
        any = any || m;
      }
      const u64 bal = __ballot(any);
      // node n of the tile is handled by lanes [n * 64 / NPT, (n + 1) * 64 / NPT)
      uint32_t am = 0;
#pragma unroll
      for (int n = 0; n < NPT; ++n) {
        const u64 seg = NPT == 1 ? bal : (bal >> (n * (64 / NPT))) & ((1ull << (64 / NPT)) - 1);
        am |= seg != 0 ? (1u << n) : 0u;
      }
      act[k] = am;
    }
  };
  // Plane fragments and offsets of this lane's tiles in the super-tile at `base`.
  auto load_stage = [&](int base, const int (&pp)[UN], const uint32_t (&act)[UN], Frag (&af)[UN][NK],
                        float (&bv)[UN][4]) {
#pragma unroll
    for (int k = 0; k < UN; ++k) {
      const int tbk = base + (k * 4 + wave) * NPT;
      const int pos = tbk + row / R;
      const bool v = UNI ? ((act[k] >> (row / R)) & 1u) != 0 : pos < end;
      int id = pos;
      if (!UNI && has_par) id = csh ? (pp[k] << a.v.Cshift) + (pos & ((1 << a.v.Cshift) - 1))
                                           : pp[k] * a.v.C + pos % a.v.C;
      id = v ? id : 0;
      // inactive rows read node 0 (FLAT) or nothing; their results are never written
      const T* mp = mb + ((int64_t)id * R + (row % R)) * D + grp * M::EPL;
#pragma unroll
      for (int s = 0; s < NK; ++s) af[k][s] = (FLAT || v) ? M::load(mp + s * M::KPER) : M::zero();
      if constexpr (R >= 4) {
        // rows 4grp..4grp+3 of this lane belong to one node: its four offsets in one load
        const int id2 = __shfl(id, 4 * grp);
        const bool v2 = UNI ? ((act[k] >> ((4 * grp) / R)) & 1u) != 0 : tbk + (4 * grp) / R < end;
        const float4 x = (FLAT || v2) ? *(const float4*)(bb + (int64_t)id2 * R + (4 * grp) % R)
                                      : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        bv[k][0] = v2 ? x.x : -INFINITY;
        bv[k][1] = v2 ? x.y : -INFINITY;
        bv[k][2] = v2 ? x.z : -INFINITY;
        bv[k][3] = v2 ? x.w : -INFINITY;
      } else {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int r2 = 4 * grp + jj;
          const int id2 = __shfl(id, r2);
          const bool v2 = tbk + r2 / R < end;
          const float x = (FLAT || v2) ? bb[(int64_t)id2 * R + (r2 % R)] : -INFINITY;
          bv[k][jj] = v2 ? x : -INFINITY;
        }
      }
    }
  };
  // Scores of tile k of the super-tile at `base` from its plane fragments, for every column
  // tile (F8: rs holds the rows' scales, which multiply the product; unused otherwise).
  // UNI: the lane writes for a column when its node is a member of the column's unit, at
  // that unit's frontier position.
  auto score_tile = [&](int k, const Frag (&afk)[NK], const float (&bvk)[4], const float (&rs)[4], int base,
                        const bool (&memk)[NT], const int (&wposk)[NT]) {
    const int tbk = base + (k * 4 + wave) * NPT;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < NK; ++s) acc = M::mma(afk[s], qf[n][s], acc);
      float v[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float mul = F8 ? a.scale * rs[jj] : a.scale;
        v[jj] = bvk[jj] == -INFINITY ? -INFINITY : fmaf(acc[jj], mul, bvk[jj]);
      }
      float* sc = a.scores + (int64_t)u[n] * a.cap1 * GS;
      // maximum over each node's planes; rows 4*grp+jj of this lane belong to node (4*grp+jj)/R
      if (R >= 4) {
        float mx = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
        if (R >= 8) mx = fmaxf(mx, __shfl_xor(mx, 16));
        if (R >= 16) mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool writer = (R == 4) || (R == 8 && (grp & 1) == 0) || (R == 16 && grp == 0);
        const int pos = UNI ? wposk[n] : tbk + (4 * grp) / R;
        const bool wr = UNI ? memk[n] : (ok[n] && pos < end);
        if (writer && wr) {
          sc[(int64_t)pos * GS + jc[n]] = mx;
          lse_push(runM[n], runS[n], mx);
        }
      } else if (R == 2) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const float mx = fmaxf(v[2 * h2], v[2 * h2 + 1]);
          const int pos = tbk + 2 * grp + h2;
          if (ok[n] && pos < end) {
            sc[(int64_t)pos * GS + jc[n]] = mx;
            lse_push(runM[n], runS[n], mx);
          }
        }
      } else {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int pos = tbk + 4 * grp + jj;
          if (ok[n] && pos < end) {
            sc[(int64_t)pos * GS + jc[n]] = v[jj];
            lse_push(runM[n], runS[n], v[jj]);
          }
        }
      }
    }
  };

  auto compute = [&](const Frag (&af)[UN][NK], const float (&bv)[UN][4], int base, const bool (&mem)[UN][NT],
                     const int (&wpos)[UN][NT]) {
#pragma unroll
    for (int k = 0; k < UN; ++k) score_tile(k, af[k], bv[k], bv[k], base, mem[k], wpos[k]);
  };
  // F8: codes, offsets and scales of this lane's tiles in the super-tile at `base`.
  auto load_stage8 = [&](int base, const int (&pp)[UN], const uint32_t (&act)[UN], uint4 (&rw)[UN][NR],
                         float (&bv)[UN][4], float (&sv)[UN][4]) {
#pragma unroll
    for (int k = 0; k < UN; ++k) {
      const int tbk = base + (k * 4 + wave) * NPT;
      const int pos = tbk + row / R;
      const bool v = UNI ? ((act[k] >> (row / R)) & 1u) != 0 : pos < end;
      int id = pos;
      if (!UNI && has_par) id = csh ? (pp[k] << a.v.Cshift) + (pos & ((1 << a.v.Cshift) - 1))
                                           : pp[k] * a.v.C + pos % a.v.C;
      id = v ? id : 0;
      if constexpr (F4) {
        // the lane's d/4 codes (d/8 bytes) and the scale of the block they lie in
        const int64_t rw4 = (int64_t)id * R + (row % R);
        const uint8_t* cp = m8 + rw4 * (D / 2) + grp * (D / 8);
        if constexpr (D == 128) {
          rw[k][0] = *(const uint4*)cp;
        } else {
          const uint2 q2 = *(const uint2*)cp;
          rw[k][0] = make_uint4(q2.x, q2.y, 0u, 0u);
        }
        sv[k][0] = fp4_scale(sb4[rw4 * (D / 32) + (grp * (D / 4)) / 32]);
      } else {
        const uint8_t* cp = m8 + ((int64_t)id * R + (row % R)) * D + grp * (D / 4);
#pragma unroll
        for (int i = 0; i < NR; ++i) rw[k][i] = (FLAT || v) ? *(const uint4*)(cp + 16 * i) : make_uint4(0u, 0u, 0u, 0u);
      }
      if constexpr (R >= 4) {
        const int id2 = __shfl(id, 4 * grp);
        const bool v2 = UNI ? ((act[k] >> ((4 * grp) / R)) & 1u) != 0 : tbk + (4 * grp) / R < end;
        const int64_t o = (int64_t)id2 * R + (4 * grp) % R;
        const float4 b4 = (FLAT || v2) ? *(const float4*)(bb + o)
                                       : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        bv[k][0] = v2 ? b4.x : -INFINITY;
        bv[k][1] = v2 ? b4.y : -INFINITY;
        bv[k][2] = v2 ? b4.z : -INFINITY;
        bv[k][3] = v2 ? b4.w : -INFINITY;
        if constexpr (F8) {
          const float4 s4 = (FLAT || v2) ? *(const float4*)(sb + o) : make_float4(0.f, 0.f, 0.f, 0.f);
          sv[k][0] = s4.x; sv[k][1] = s4.y; sv[k][2] = s4.z; sv[k][3] = s4.w;
        }
      } else {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int r2 = 4 * grp + jj;
          const int id2 = __shfl(id, r2);
          const bool v2 = tbk + r2 / R < end;
          const int64_t o = (int64_t)id2 * R + (r2 % R);
          const float x = (FLAT || v2) ? bb[o] : -INFINITY;
          bv[k][jj] = v2 ? x : -INFINITY;
          if constexpr (F8) sv[k][jj] = (FLAT || v2) ? sb[o] : 0.0f;
        }
      }
    }
  };
  // F8: decode the codes (lane k-slots s*8 .. s*8+7 of its d/4 codes per matrix step),
  // then score as the bf16 path does with the row scale in the multiplier.  F4: decode with
  // the block scale folded in (the multiplier is the logit scale alone).
  auto compute8 = [&](const uint4 (&rw)[UN][NR], const float (&bv)[UN][4], const float (&sv)[UN][4], int base,
                      const bool (&mem)[UN][NT], const int (&wpos)[UN][NT]) {
    if constexpr (LP) {
#pragma unroll
      for (int k = 0; k < UN; ++k) {
        Frag afk[NK];
#pragma unroll
        for (int s = 0; s < NK; ++s) {
          if constexpr (F4) {
            const uint4 q4 = rw[k][0];
            const uint32_t wd = s == 0 ? q4.x : (s == 1 ? q4.y : (s == 2 ? q4.z : q4.w));
            afk[s] = fp4x8_to_bf16(wd, sv[k][0]);
          } else {
            const uint4 q4 = rw[k][s / 2];
            afk[s] = (s & 1) ? fp8x8_to_bf16(q4.z, q4.w) : fp8x8_to_bf16(q4.x, q4.y);
          }
        }
        score_tile(k, afk, bv[k], sv[k], base, mem[k], wpos[k]);
      }
    }
  };

  // Software pipeline over the workgroup's super-tiles: while one is scored, the planes of
  // the next and the parent entries of the one after are in flight.  The two register
  // buffers alternate by unrolling the loop twice.
  int ppA[UN], ppB[UN];
  u64 rkA[UN][NT], rkB[UN][NT];
  bool mA[UN][NT], mB[UN][NT];
  int wA[UN][NT], wB[UN][NT];
  uint32_t acA[UN], acB[UN];
  float bvA[UN][4], bvB[UN][4];
  fetch_par(start, ppA, rkA);
  fetch_par(start + step, ppB, rkB);
  if constexpr (UNI) members(start, rkA, mA, wA, acA);
  if constexpr (LP) {
    uint4 rwA[UN][NR], rwB[UN][NR];
    float svA[UN][4], svB[UN][4];
    if (start < end) load_stage8(start, ppA, acA, rwA, bvA, svA);
    for (int base = start; base < end;) {
      if constexpr (UNI) members(base + step, rkB, mB, wB, acB);
      fetch_par(base + 2 * step, ppA, rkA);
      load_stage8(base + step, ppB, acB, rwB, bvB, svB);
      compute8(rwA, bvA, svA, base, mA, wA);
      base += step;
      if (base >= end) break;
      if constexpr (UNI) members(base + step, rkA, mA, wA, acA);
      fetch_par(base + 2 * step, ppB, rkB);
      load_stage8(base + step, ppA, acA, rwA, bvA, svA);
      compute8(rwB, bvB, svB, base, mB, wB);
      base += step;
    }
  } else {
    Frag afA[UN][NK], afB[UN][NK];
    if (start < end) load_stage(start, ppA, acA, afA, bvA);
    for (int base = start; base < end;) {
      if constexpr (UNI) members(base + step, rkB, mB, wB, acB);
      fetch_par(base + 2 * step, ppA, rkA);
      load_stage(base + step, ppB, acB, afB, bvB);
      compute(afA, bvA, base, mA, wA);
      base += step;
      if (base >= end) break;
      if constexpr (UNI) members(base + step, rkA, mA, wA, acA);
      fetch_par(base + 2 * step, ppB, rkB);
      load_stage(base + step, ppA, acA, afA, bvA);
      compute(afB, bvB, base, mB, wB);
      base += step;
    }
  }
  // per-column (max, sum exp) of this workgroup: lanes of one column, then the 4 waves
  __shared__ float sM[4][16 * NT], sS[4][16 * NT];
  __shared__ int sU[16 * NT], sJ[16 * NT];
  __shared__ bool sOk[16 * NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    float rM = runM[n], rS = runS[n];
    float M2 = __shfl_xor(rM, 16), S2 = __shfl_xor(rS, 16);
    lse_merge(rM, rS, M2, S2);
    M2 = __shfl_xor(rM, 32);
    S2 = __shfl_xor(rS, 32);
    lse_merge(rM, rS, M2, S2);
    if (grp == 0) { sM[wave][16 * n + row] = rM; sS[wave][16 * n + row] = rS; }
    if (wave == 0 && grp == 0) { sU[16 * n + row] = u[n]; sJ[16 * n + row] = jc[n]; sOk[16 * n + row] = ok[n]; }
  }
  __syncthreads();
  const int c = threadIdx.x;
  if (c < 16 * NT && sOk[c]) {
    float Mx = sM[0][c], Sx = sS[0][c];
    for (int w = 1; w < 4; ++w) lse_merge(Mx, Sx, sM[w][c], sS[w][c]);
    float* pp = a.part + (((int64_t)sU[c] * a.W + blockIdx.x) * G + sJ[c]) * 2;
    pp[0] = Mx;
    pp[1] = Sx;
  }
}

// ------------------------------------------------------------------------ shared selection
//
// The selection kernels run a handful of workgroups each, so their time is the length of
// their dependent instruction and memory chains: loads are issued in batches, reductions
// run across all threads at once, and no step walks a list serially.

// Per-head log-sum-exp over the frontier from the W <= 512 scoring partials of unit u,
// into lse[0..G), with 256 threads: 16 per head, every partial loaded at once.  Fixed
// combination order: every workgroup calling this gets the same bits.
__device__ __forceinline__ void frontier_lse256(const float* part, int W, int G, int u, float* lse) {
  const int h = threadIdx.x >> 4, j = threadIdx.x & 15;
  float2 pv[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const int i = j + 16 * k;
    pv[k] = (h < G && i < W) ? *(const float2*)(part + (((int64_t)u * W + i) * G + h) * 2)
                             : make_float2(-INFINITY, 0.0f);
  }
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < 32; ++k) M = fmaxf(M, pv[k].x);
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 16));
  float S = 0.0f;
  if (M != -INFINITY) {
#pragma unroll
    for (int k = 0; k < 32; ++k) S += pv[k].x == -INFINITY ? 0.0f : pv[k].y * zexp(pv[k].x - M);
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) S += __shfl_xor(S, o, 16);
  if (h < G && j == 0) lse[h] = M == -INFINITY ? -INFINITY : M + zlog(S);
}

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

// A key range [lo, hi] is cut into slices of 2^s consecutive key values, s the smallest
// shift that leaves at most NB slices; the slice of a key is a shift (monotone in key).
constexpr int NB_LOG2 = 10;
static_assert(NB == 1 << NB_LOG2, "NB is a power of two");

__device__ __forceinline__ int range_shift(uint32_t lo, uint32_t hi) {
  const uint32_t d = hi - lo;
  const int bits = d == 0u ? 0 : 32 - __clz((int)d);
  return bits > NB_LOG2 ? bits - NB_LOG2 : 0;
}

__device__ __forceinline__ uint32_t range_bin(uint32_t key, uint32_t lo, int shift) { return (key - lo) >> shift; }

// Key range of slice b of [lo, hi].
__device__ __forceinline__ void slice_range(uint32_t lo, uint32_t hi, uint32_t b, uint32_t* nlo, uint32_t* nhi) {
  const int shift = range_shift(lo, hi);
  const u64 a = (u64)lo + ((u64)b << shift);
  const u64 e = a + ((u64)1 << shift) - 1;
  *nlo = (uint32_t)a;
  *nhi = e < (u64)hi ? (uint32_t)e : hi;
}

// Key window of the fine histogram: 16 binades of fp32 masses, from 2^-12/n to 16/n
// around the uniform mass 1/n, in NB slices of 1/64 binade.  Keys below it hold less
// than 2^-12 of the total mass together.
constexpr int FINE_SHIFT = 27 - NB_LOG2;
__device__ __forceinline__ void fine_window(int n, uint32_t* lo, uint32_t* hi) {
  const uint32_t ref = __float_as_uint(1.0f / (float)n);
  *lo = ref - (12u << 23);
  *hi = *lo + (1u << 27) - 1u;
}

// Ties at the cut all carry the same mass: the fewest that reach T, ceil((T - above) / mt).
// Both operands are below 2^42, so the double quotient is within one of the answer and
// one exact integer correction each way settles it.
__device__ __forceinline__ uint32_t ties_to_take(uint32_t tau, u64 T, u64 above) {
  const u64 mt = fx_mass(tau) > 0 ? fx_mass(tau) : 1;  // the cut element always carries mass
  const u64 need = T - above;
  u64 q = (u64)((double)need / (double)mt);
  if (q * mt < need) ++q;
  if (q > 0 && (q - 1) * mt >= need) --q;
  return (uint32_t)q;
}

__device__ __forceinline__ u64 target_of(float p, u64 total) {
  u64 T = (u64)ceil((double)p * (double)total);  // c >= p W  <=>  c >= ceil(p W) for integer c
  if (T < 1) T = 1;
  if (T > total) T = total;
  return T;
}

// Four keys at pos (a multiple of 4) from a buffer of ncap readable keys (a multiple of 4,
// at least 4): the address is clamped, so the load never branches; callers mask by count.
__device__ __forceinline__ uint4 load4c(const uint32_t* k, int pos, int ncap) {
  return *(const uint4*)(k + min(pos, ncap - 4));
}


// ------------------------------------------------------------ small-frontier selection
//
// A frontier of at most WN nodes is selected by a workgroup of SSEL = 256 threads, thread
// t holding positions t, t + 256, t + 512, t + 768.  Every load of a thread is issued at once
// (parent ids and score rows at positions clamped to the level's capacity, so none waits
// for the frontier size).  The per-head log-sum-exp over the frontier is a maximum then a
// sum, each over the thread's positions, the wave (DPP and lane swaps: every lane gets the
// same bits) and the four waves in order; then the mass keys and their fixed-point total.
// The cut: a histogram of NB slices of the key range (LDS atomics), a scan over the threads
// from the heaviest slice down for the crossing slice, and its keys ranked by one wave (at
// most 64, one per lane); more than 64 keys in the slice narrow the range to it and the
// histogram is repeated.  The kept nodes are written in position order: each wave counts
// its 256 positions (ballots), then writes them after the earlier waves' counts.  The rule
// is that of the multi-wave selections: keep keys above the cut key tau, and keys equal to
// tau up to the position tie_last.

constexpr int SSEL = 256;            // threads of the small selection
constexpr int SSPT = WN / SSEL;      // frontier positions per thread
static_assert(SSPT == 4 && NB == 4 * SSEL, "four positions and four histogram slices per thread");

__device__ void wave_select(const Level& v, int u, int capF, const float* scores, int64_t sstride, int G, float p,
                            int keep_all, WaveSh& sh, int& nF_out, int& nk_out, int& nx_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const u64 lt = (1ull << lane) - 1ull;  // lanes below this one
  __shared__ float s_red[SSEL / 64][16];
  __shared__ uint32_t s_min[SSEL / 64], s_max[SSEL / 64];
  __shared__ u64 s_tot[SSEL / 64], s_scan[SSEL / 64];
  __shared__ uint32_t s_bin, s_nc, s_tau;
  __shared__ int s_tie;
  __shared__ u64 s_above;
  __shared__ int s_cnt[SSEL / 64], s_last;
  // every load at once: the frontier size, parent ids and score rows (clamped positions)
  const int nF = frontier_size(v, u);
  const int nchild = child_nodes(v, u);
  const int32_t* par = v.parent ? v.parent + (int64_t)u * v.cap_parent : nullptr;
  const int GS = score_stride(G);
  const float* sc = scores + (int64_t)u * sstride * GS;
  const int cmax = max(capF, 1) - 1;
  int pid[SSPT];
  float4 sv[SSPT][4];
#pragma unroll
  for (int k = 0; k < SSPT; ++k) {
    const int pc = min(tid + SSEL * k, cmax);
    pid[k] = par ? par[v.Cshift >= 0 ? pc >> v.Cshift : pc / v.C] : 0;
    load_scores(sc + (int64_t)pc * GS, G, sv[k]);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    sh.hcnt[tid + SSEL * e] = 0;
    sh.hmass[tid + SSEL * e] = 0;
  }
  if (tid == 0) s_nc = 0;
  bool val[SSPT];
#pragma unroll
  for (int k = 0; k < SSPT; ++k) val[k] = tid + SSEL * k < nF;
  // per-head maximum, then sum of exp(s - max), over the frontier
  float lse[16];
#pragma unroll
  for (int h4 = 0; h4 < 4; ++h4) {
    if (4 * h4 < G) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float m = -INFINITY;
#pragma unroll
        for (int k = 0; k < SSPT; ++k) {
          const float x = j == 0 ? sv[k][h4].x : (j == 1 ? sv[k][h4].y : (j == 2 ? sv[k][h4].z : sv[k][h4].w));
          m = val[k] ? fmaxf(m, x) : m;
        }
        m = wave_max(m);
        if (lane == 0) s_red[wave][4 * h4 + j] = m;
      }
    }
  }
  __syncthreads();
  float hmax[16];
#pragma unroll
  for (int h = 0; h < 16; ++h) {
    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < SSEL / 64; ++w) m = fmaxf(m, h < G ? s_red[w][h] : -INFINITY);
    hmax[h] = m;
  }
  __syncthreads();  // s_red is reused for the sums
#pragma unroll
  for (int h4 = 0; h4 < 4; ++h4) {
    if (4 * h4 < G) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float M = hmax[4 * h4 + j];
        float e = 0.0f;
#pragma unroll
        for (int k = 0; k < SSPT; ++k) {
          const float x = j == 0 ? sv[k][h4].x : (j == 1 ? sv[k][h4].y : (j == 2 ? sv[k][h4].z : sv[k][h4].w));
          e += (val[k] && x != -INFINITY) ? zexp(x - M) : 0.0f;
        }
        e = wave_sum(e);
        if (lane == 0) s_red[wave][4 * h4 + j] = e;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 16; ++h) {
    float S = 0.0f;
#pragma unroll
    for (int w = 0; w < SSEL / 64; ++w) S += h < G ? s_red[w][h] : 0.0f;
    lse[h] = (h < G && hmax[h] != -INFINITY) ? hmax[h] + zlog(S) : 0.0f;
  }
  // node ids and mass keys by position; their range and fixed-point total
  const float invG = 1.0f / (float)G;
  uint32_t key[SSPT];
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  u64 tot = 0;
#pragma unroll
  for (int k = 0; k < SSPT; ++k) {
    const int pos = tid + SSEL * k;
    key[k] = mass_key(sv[k], lse, G, invG);
    if (val[k]) {
      sh.fid[pos] = par ? (v.Cshift >= 0 ? (pid[k] << v.Cshift) + (pos & ((1 << v.Cshift) - 1))
                                         : pid[k] * v.C + pos % v.C)
                        : pos;
      sh.keys[pos] = key[k];
      kmin = min(kmin, key[k]);
      kmax = max(kmax, key[k]);
      tot += fx_mass(key[k]);
    }
  }
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  tot = wave_sum_u64(tot);
  if (lane == 0) { s_min[wave] = kmin; s_max[wave] = kmax; s_tot[wave] = tot; }
  __syncthreads();
  kmin = s_min[0]; kmax = s_max[0]; tot = s_tot[0];
#pragma unroll
  for (int w = 1; w < SSEL / 64; ++w) { kmin = min(kmin, s_min[w]); kmax = max(kmax, s_max[w]); tot += s_tot[w]; }
  const bool all = keep_all || nF == 0 || tot == 0;  // tot 0: every mass rounds to zero
  uint32_t tau = 0;
  int tie_last = 0x7FFFFFFF;
  if (!all) {
    const u64 T = target_of(p, tot);
    uint32_t lo = kmin, hi = kmax;
    u64 above = 0;
    for (int round = 0;; ++round) {
      const int shift = range_shift(lo, hi);
      if (round > 0) {  // a narrowed range: a fresh histogram
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sh.hcnt[tid + SSEL * e] = 0;
          sh.hmass[tid + SSEL * e] = 0;
        }
        if (tid == 0) s_nc = 0;
        __syncthreads();
      }
#pragma unroll
      for (int k = 0; k < SSPT; ++k) {
        if (val[k] && key[k] >= lo && key[k] <= hi) {
          const uint32_t bn = range_bin(key[k], lo, shift);
          atomicAdd(&sh.hcnt[bn], 1u);
          atomicAdd(&sh.hmass[bn], fx_mass(key[k]));
        }
      }
      __syncthreads();
      // thread t owns slices NB-1-4t .. NB-4-4t (heaviest first); the mass above them is a
      // prefix over the threads
      u64 m4[4], msum = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        m4[e] = sh.hmass[NB - 1 - 4 * tid - e];
        msum += m4[e];
      }
      u64 inc = msum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const u64 y = __shfl_up(inc, o);
        inc += lane >= o ? y : 0;
      }
      if (lane == 63) s_scan[wave] = inc;
      __syncthreads();
      u64 before = above + inc - msum;
#pragma unroll
      for (int w = 0; w < SSEL / 64; ++w) before += w < wave ? s_scan[w] : 0;
      if (before < T && before + msum >= T) {  // exactly one thread
        u64 run = before;
        int f = 3;
        for (int e = 0; e < 4; ++e) {
          if (run + m4[e] >= T) { f = e; break; }
          run += m4[e];
        }
        s_bin = (uint32_t)(NB - 1 - 4 * tid - f);
        s_above = run;
      }
      __syncthreads();
      const uint32_t bin = s_bin;
      above = s_above;
      const uint32_t cnt = sh.hcnt[bin];
      uint32_t nlo, nhi;
      slice_range(lo, hi, bin, &nlo, &nhi);
      if (cnt <= 64u) {
        // the slice's keys, by all threads, in any order
#pragma unroll
        for (int k = 0; k < SSPT; ++k) {
          if (val[k] && key[k] >= nlo && key[k] <= nhi) {
            const uint32_t slot = atomicAdd(&s_nc, 1u);
            sh.ckey[slot] = key[k];
            sh.cpos[slot] = (uint32_t)(tid + SSEL * k);
          }
        }
        __syncthreads();
        if (wave == 0) {
          const bool mine = lane < (int)cnt;
          const uint32_t mk = sh.ckey[mine ? lane : 0], mp = sh.cpos[mine ? lane : 0];
          const u64 mm = fx_mass(mk);
          u64 bf = above;
          for (int j = 0; j < (int)cnt; ++j) {  // (readlane returns int: every word widened unsigned)
            const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)mk, j);
            const uint32_t qj = (uint32_t)__builtin_amdgcn_readlane((int)mp, j);
            const u64 mj = ((u64)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(mm >> 32), j) << 32) |
                           (u64)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)mm, j);
            bf += (kj > mk || (kj == mk && qj < mp)) ? mj : 0;
          }
          const u64 c = __ballot(mine && bf < T && bf + mm >= T);
          const int cl = c ? __ffsll((unsigned long long)c) - 1 : 0;
          if (lane == 0) {
            s_tau = (uint32_t)__builtin_amdgcn_readlane((int)mk, cl);
            s_tie = __builtin_amdgcn_readlane((int)mp, cl);
          }
        }
        __syncthreads();
        tau = s_tau;
        tie_last = s_tie;
        break;
      }
      if (nhi <= nlo) {
        // more than 64 keys of one value: the first n_take of them in position order
        const uint32_t n_take = ties_to_take(nlo, T, above);
        tau = nlo;
        if (n_take < cnt) {
          if (wave == 0) {
            uint32_t seen = 0;
            int tl = 0;
            for (int r0 = 0; r0 < nF; r0 += 64) {
              const int pos = r0 + lane;
              const bool eq = pos < nF && sh.keys[min(pos, nF - 1)] == tau;
              const u64 b = __ballot(eq);
              const uint32_t pc = (uint32_t)__popcll(b);
              if (seen + pc >= n_take) {  // the n_take-th equal key lies in this row
                const uint32_t rank = seen + (uint32_t)__popcll(b & lt);
                const u64 w = __ballot(eq && rank == n_take - 1);
                tl = r0 + (__ffsll((unsigned long long)w) - 1);
                break;
              }
              seen += pc;
            }
            if (lane == 0) s_tie = tl;
          }
          __syncthreads();
          tie_last = s_tie;
        }
        break;
      }
      lo = nlo;
      hi = nhi;
    }
  }
  // the kept nodes in position order: wave w writes positions [256 w, 256 w + 256) after the
  // kept counts of the waves before it
  bool kp[SSPT];
  int cnt_w = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int pos = SSEL * wave + 64 * r + lane;
    const uint32_t k = sh.keys[min(pos, max(nF, 1) - 1)];
    kp[r] = pos < nF && (all || k > tau || (k == tau && pos <= tie_last));
    cnt_w += __popcll(__ballot(kp[r]));
  }
  if (lane == 0) s_cnt[wave] = cnt_w;
  if (tid == 0) s_last = -1;
  __syncthreads();
  int base = 0, nk = 0;
#pragma unroll
  for (int w = 0; w < SSEL / 64; ++w) {
    base += w < wave ? s_cnt[w] : 0;
    nk += s_cnt[w];
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int pos = SSEL * wave + 64 * r + lane;
    const u64 b = __ballot(kp[r]);
    if (kp[r]) {
      const int id = sh.fid[pos];
      sh.kept[base + __popcll(b & lt)] = id;
      if (pos == nF - 1) s_last = id;
    }
    base += __popcll(b);
  }
  __syncthreads();
  const int last_id = s_last;
  nF_out = nF;
  nk_out = nk;
  nx_out = last_id >= 0 ? next_frontier(nk, last_id, v.C, nchild) : v.C * nk;
}

struct WaveArgs {
  Level v;
  const float* scores;    // [U][sstride][score row]
  int64_t sstride;
  int G;
  float p;
  int keep_all;
  int32_t* kept;          // [U][capl]
  int64_t capl;
  int32_t* nF_out;        // [U]
  int32_t* kept_count;    // [U]
  int32_t* next_nF;       // [U]; null at level 1
};

// A level of at most WN nodes whose selection is not run by the next level's scoring
// launch (level 1, or routes of grouped units): one workgroup of SSEL threads per unit.
__global__ __launch_bounds__(SSEL) void zha_select_wave_kernel(WaveArgs a) {
  __shared__ WaveSh sh;
  const int u = blockIdx.x;
  int nF, nk, nx;
  wave_select(a.v, u, (int)a.capl, a.scores, a.sstride, a.G, a.p, a.keep_all, sh, nF, nk, nx);
  int32_t* kp = a.kept + (int64_t)u * a.capl;
  for (int i = threadIdx.x; i < nk; i += SSEL) kp[i] = sh.kept[i];
  if (threadIdx.x == 0) {
    a.nF_out[u] = nF;
    a.kept_count[u] = nk;
    if (a.next_nF) a.next_nF[u] = nx;
  }
}

// Selection state of one workgroup (LDS).  ST = 512 threads: two waves per SIMD keep the
// throughput phases at full issue rate while a serial step waits only on its own
// instruction latency.  Each thread owns two histogram bins.
constexpr int ST = 512;
constexpr int BPT = NB / ST;             // histogram bins per thread
static_assert(BPT == 2, "two bins per thread");
constexpr int RMAX = 64;                 // crossing-slice keys resolved by ranking

struct CutSh {
  uint32_t hcnt[NB];
  u64 hmass[NB];
  uint32_t rkey[RMAX];
  uint32_t rpos[RMAX];
  u64 rmass[RMAX];
  u64 red64[ST / 64];
  uint32_t scan[ST / 64];
  uint32_t bin, ncand, tau;
  int lastpos, tie_last;
  u64 above;
};

__device__ __forceinline__ void hist_clear(CutSh& sh) {
#pragma unroll
  for (int e = 0; e < BPT; ++e) {
    sh.hcnt[threadIdx.x + ST * e] = 0;
    sh.hmass[threadIdx.x + ST * e] = 0;
  }
}

// Histogram over the slices of [lo, hi] of the keys src[0, n) (keys outside are skipped);
// keys (16-byte aligned) are read 16 per thread per round trip.
__device__ __forceinline__ void hist_keys(CutSh& sh, const uint32_t* src, int n, int ncap, uint32_t lo, uint32_t hi) {
  const int shift = range_shift(lo, hi);
  for (int base = 16 * threadIdx.x; base < n; base += 16 * ST) {
    uint4 kv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) kv[j] = load4c(src, base + 4 * j, ncap);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t k4[4] = {kv[j].x, kv[j].y, kv[j].z, kv[j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t k = k4[e];
        if (base + 4 * j + e < n && k >= lo && k <= hi) {
          const uint32_t bn = range_bin(k, lo, shift);
          atomicAdd(&sh.hcnt[bn], 1u);
          atomicAdd(&sh.hmass[bn], fx_mass(k));
        }
      }
    }
  }
}

// The slice in which the mass, accumulated from the heaviest slice down on top of
// sh.above, reaches T: thread t owns slices NB-1-2t and NB-2-2t, and a workgroup scan
// gives every slice the mass above it.  Sets sh.bin and sh.above.
__device__ __forceinline__ void find_bin(CutSh& sh, u64 T) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const u64 above0 = sh.above;
  const u64 m0 = sh.hmass[NB - 1 - 2 * tid], m1 = sh.hmass[NB - 2 - 2 * tid];
  const u64 m = m0 + m1;
  u64 inc = m;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const u64 y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  if (lane == 63) sh.red64[wave] = inc;
  __syncthreads();
  u64 run = above0 + inc - m;
#pragma unroll
  for (int w = 0; w < ST / 64; ++w) run += w < wave ? sh.red64[w] : 0;
  __syncthreads();
  if (run < T && run + m0 >= T) {
    sh.bin = (uint32_t)(NB - 1 - 2 * tid);
    sh.above = run;
  } else if (run + m0 < T && run + m >= T) {
    sh.bin = (uint32_t)(NB - 2 - 2 * tid);
    sh.above = run + m0;
  }
  __syncthreads();
}

// LDS versions (keys in LDS, position = index): four keys per thread in flight, one
// short predicated body per key.
__device__ __forceinline__ void hist_keys_lds(CutSh& sh, const uint32_t* keys, int n, uint32_t lo, uint32_t hi) {
  const int shift = range_shift(lo, hi);
  for (int i0 = threadIdx.x; i0 < n; i0 += 4 * ST) {
    uint32_t k4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) k4[e] = keys[min(i0 + ST * e, n - 1)];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t k = k4[e];
      if (i0 + ST * e < n && k >= lo && k <= hi) {
        const uint32_t bn = range_bin(k, lo, shift);
        atomicAdd(&sh.hcnt[bn], 1u);
        atomicAdd(&sh.hmass[bn], fx_mass(k));
      }
    }
  }
}

// Positions are pos[i] (candidates carrying their frontier positions) or i itself (pos null).
__device__ __forceinline__ void gather_slice_lds(CutSh& sh, const uint32_t* keys, const uint32_t* pos, int n,
                                                 uint32_t lo, uint32_t hi) {
  if (threadIdx.x == 0) sh.ncand = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  for (int i0 = threadIdx.x - lane; i0 < n; i0 += 4 * ST) {  // uniform per wave
    uint32_t k4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) k4[e] = keys[min(i0 + lane + ST * e, n - 1)];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = i0 + lane + ST * e;
      const bool hit = i < n && k4[e] >= lo && k4[e] <= hi;
      const u64 m = __ballot(hit);  // one reservation per wave
      if (m) {
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&sh.ncand, (uint32_t)__popcll(m));
        base = __shfl(base, 0);
        if (hit) {
          const uint32_t slot = base + (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
          sh.rkey[slot] = k4[e];
          sh.rpos[slot] = pos ? pos[i] : (uint32_t)i;
        }
      }
    }
  }
  __syncthreads();
}

// The exact cut among the c <= RMAX keys in sh.rkey/rpos, sh.above being the mass of
// every key above them: each candidate adds up the masses of the candidates ordered
// before it (mass descending, position ascending); the one whose own mass makes the
// running total reach T is the last node kept.  Sets sh.tau and sh.tie_last.
__device__ __forceinline__ void rank_cut(CutSh& sh, int c, u64 T) {
  const int tid = threadIdx.x;
  if (tid < c) sh.rmass[tid] = fx_mass(sh.rkey[tid]);
  __syncthreads();
  if (tid < c) {
    const uint32_t mk = sh.rkey[tid], mp = sh.rpos[tid];
    u64 before = sh.above;
#pragma unroll 8
    for (int j = 0; j < c; ++j) {
      const uint32_t k = sh.rkey[j], q = sh.rpos[j];
      before += (k > mk || (k == mk && q < mp)) ? sh.rmass[j] : 0;
    }
    if (before < T && before + sh.rmass[tid] >= T) {
      sh.tau = mk;
      sh.tie_last = (int)mp;
    }
  }
  __syncthreads();
}

// Position of the n-th (0-based) key equal to tau in position order, by counting scans.
__device__ __forceinline__ int nth_tie_scan(CutSh& sh, const uint32_t* keys, int nF, int ncap, uint32_t tau,
                                            uint32_t n) {
  uint32_t seen = 0;
  int found = -1;
  for (int base = 0; base < nF && found < 0; base += 4 * ST) {
    const int p0 = base + 4 * threadIdx.x;
    const uint4 kv = load4c(keys, p0, ncap);
    const uint32_t k4[4] = {kv.x, kv.y, kv.z, kv.w};
    uint32_t ne = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) ne += (p0 + e < nF && k4[e] == tau) ? 1u : 0u;
    uint32_t tot;
    uint32_t ex = block_excl_scan<ST>(ne, &tot, sh.scan) + seen;
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

// The cut of LDS keys[0, n) given a histogram of [lo, hi] in sh: narrow the range until
// the crossing slice holds at most RMAX keys, then rank them.  Positions are pos[i] (LDS
// candidates; ties of one value are then split by a scan of the global keys gkeys[0, gn)
// in position order) or i itself (pos null: keys is the whole frontier in position order).
__device__ __forceinline__ void resolve_cut_lds(CutSh& sh, const uint32_t* keys, const uint32_t* pos, int n,
                                                uint32_t lo, uint32_t hi, u64 T, const uint32_t* gkeys, int gn,
                                                int gcap, uint32_t* tau, int* tie_last) {
  for (;;) {
    find_bin(sh, T);
    uint32_t nlo, nhi;
    slice_range(lo, hi, sh.bin, &nlo, &nhi);
    const uint32_t cnt = sh.hcnt[sh.bin];
    if (cnt <= (uint32_t)RMAX) {
      gather_slice_lds(sh, keys, pos, n, nlo, nhi);
      rank_cut(sh, (int)cnt, T);
      *tau = sh.tau;
      *tie_last = sh.tie_last;
      return;
    }
    if (nhi <= nlo) {  // more than RMAX keys of one value
      const uint32_t n_take = ties_to_take(nlo, T, sh.above);
      *tau = nlo;
      if (n_take >= cnt) *tie_last = 0x7FFFFFFF;
      else if (pos) *tie_last = nth_tie_scan(sh, gkeys, gn, gcap, nlo, n_take - 1);
      else *tie_last = nth_tie_scan(sh, keys, n, SMALL_NODES, nlo, n_take - 1);
      return;
    }
    lo = nlo;
    hi = nhi;
    hist_clear(sh);
    __syncthreads();
    hist_keys_lds(sh, keys, n, lo, hi);
    __syncthreads();
  }
}

// gather_slice over keys in global memory (position = index): 64 keys per thread per
// round trip, so a unit's tens of thousands of keys take one or two.
__device__ __forceinline__ void gather_slice_global(CutSh& sh, const uint32_t* src, int n, int ncap, uint32_t lo,
                                                    uint32_t hi, uint32_t* dk, uint32_t* dp) {
  if (threadIdx.x == 0) sh.ncand = 0;
  __syncthreads();
  for (int base = 64 * threadIdx.x; base < n; base += 64 * ST) {
    uint4 kv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) kv[j] = load4c(src, base + 4 * j, ncap);
    // matches as a bit mask (no per-key branch), one reservation per thread, then only
    // the matching keys are written
    u64 mask = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t k4[4] = {kv[j].x, kv[j].y, kv[j].z, kv[j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool hit = base + 4 * j + e < n && k4[e] >= lo && k4[e] <= hi;
        mask |= hit ? (u64)1 << (4 * j + e) : 0;
      }
    }
    if (mask) {
      uint32_t slot = atomicAdd(&sh.ncand, (uint32_t)__popcll(mask));
      while (mask) {
        const int b = __ffsll((unsigned long long)mask) - 1;
        mask &= mask - 1;
        dk[slot] = src[base + b];  // re-read (cached): a register array cannot be indexed by b
        dp[slot] = (uint32_t)(base + b);
        ++slot;
      }
    }
  }
  __syncthreads();
}

// The cut of keys[0, n) (position = index, global memory) given a histogram of [lo, hi]
// in sh (sh.above: mass above the range, T within the range).  The range narrows NB-fold
// per pass until the crossing slice holds at most RMAX keys, which are ranked.  Once the
// crossing slice fits the LDS candidate buffer (ck/cp, ncap entries) its keys and
// positions move there and the LDS resolver finishes.  A slice of more than RMAX equal
// keys is split by position.  Returns tau and the position of the last kept key equal to tau.
__device__ __forceinline__ void resolve_cut(CutSh& sh, const uint32_t* keys, int n, int kcap, uint32_t lo, uint32_t hi,
                                            u64 T, uint32_t* ck, uint32_t* cp, int ncap, uint32_t* tau, int* tie_last) {
  for (;;) {
    find_bin(sh, T);
    uint32_t nlo, nhi;
    slice_range(lo, hi, sh.bin, &nlo, &nhi);
    const uint32_t cnt = sh.hcnt[sh.bin];
    if (cnt <= (uint32_t)RMAX) {
      gather_slice_global(sh, keys, n, kcap, nlo, nhi, sh.rkey, sh.rpos);
      rank_cut(sh, (int)cnt, T);
      *tau = sh.tau;
      *tie_last = sh.tie_last;
      return;
    }
    if (nhi <= nlo) {  // more than RMAX keys of one value
      const uint32_t n_take = ties_to_take(nlo, T, sh.above);
      *tau = nlo;
      *tie_last = n_take < cnt ? nth_tie_scan(sh, keys, n, kcap, nlo, n_take - 1) : 0x7FFFFFFF;
      return;
    }
    if (cnt <= (uint32_t)ncap) {
      gather_slice_global(sh, keys, n, kcap, nlo, nhi, ck, cp);
      hist_clear(sh);
      __syncthreads();
      hist_keys_lds(sh, ck, (int)cnt, nlo, nhi);
      __syncthreads();
      resolve_cut_lds(sh, ck, cp, (int)cnt, nlo, nhi, T, keys, n, kcap, tau, tie_last);
      return;
    }
    lo = nlo;
    hi = nhi;
    hist_clear(sh);
    __syncthreads();
    hist_keys(sh, keys, n, kcap, lo, hi);
    __syncthreads();
  }
}

// --------------------------------------------------------------------------- small levels

struct SmallArgs {
  Level v;
  const float* scores;    // [U][cap1][score row]
  int64_t cap1;
  const float* part;      // [U][W][G][2] scoring partials
  int W;                  // <= 512
  int32_t* kept;          // [U][capl]
  int64_t capl;           // <= SMALL_NODES
  int npar;               // parent ids read: ceil(capl / C) <= SMALL_NODES / 2
  int32_t* nF_out;        // this level's frontier counts [U]
  int32_t* kept_count;    // [U]
  int32_t* next_nF;       // next level's frontier counts [U]; null at level 1
  int G;
  float p;
  int keep_all;
  u64* krank;             // union routes: [U][capl] (stamp << 32) | rank of each kept node; else null
  const uint32_t* route_ctr;  // the route's stamp
  uint32_t* uflag;        // union routes at level 1: [groups][ufstride] stamp of every kept chunk
  int64_t ufstride;
  int hr, Hkv, Tq, TS, NTC;  // routing-unit numbering and union groups (for the unit's group)
};

constexpr int SBATCH = 8;     // frontier positions per thread per load batch

struct SmallSh {
  CutSh cut;
  alignas(16) uint32_t keys[SMALL_NODES];
  int32_t par[SMALL_NODES / 2];   // kept parents (C >= 2)
  uint32_t mn[ST / 64], mx[ST / 64];
  float lse[16];
  int last_kept_id;
};

// Whole selection of a frontier of at most SMALL_NODES nodes in one workgroup: every
// global read (scoring partials, parent ids, scores) is issued before any result is
// needed; the masses live in LDS; one histogram over the key range finds the crossing
// slice, whose keys are ranked; the kept ids are written in order.
__global__ __launch_bounds__(ST) void zha_select_small_kernel(SmallArgs a) {
  __shared__ SmallSh sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int u = blockIdx.x;
  const int G = a.G;
  const int nmax = (int)a.capl;  // >= 1
  const int nF = frontier_size(a.v, u);
  const int nchild = a.next_nF ? child_nodes(a.v, u) : 0;  // loaded now, used at the end
  const uint32_t stamp = a.krank ? a.route_ctr[0] : 0u;
  const int GS = score_stride(G);
  const float* sc = a.scores + (int64_t)u * a.cap1 * GS;
  const int32_t* gpar = a.v.parent ? a.v.parent + (int64_t)u * a.v.cap_parent : nullptr;

  // scoring partials (32 lanes per head, W <= 512), parent ids, first batch of scores:
  // all issued before the first wait, from clamped (always readable) addresses
  const int ph = tid >> 5, pl = tid & 31;
  const int phc = min(ph, G - 1);
  float2 pv[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int i = min(pl + 32 * k, a.W - 1);
    pv[k] = *(const float2*)(a.part + (((int64_t)u * a.W + i) * G + phc) * 2);
  }
  if (gpar) {
    constexpr int NPL = SMALL_NODES / 2 / ST;
    int32_t pp[NPL];
#pragma unroll
    for (int k = 0; k < NPL; ++k)
      if (ST * k < a.npar) pp[k] = gpar[min(tid + ST * k, a.npar - 1)];
#pragma unroll
    for (int k = 0; k < NPL; ++k)
      if (ST * k < a.npar) sh.par[tid + ST * k] = pp[k];
  }
  float4 sv[SBATCH][4];
#pragma unroll
  for (int k = 0; k < SBATCH; ++k)
    if (ST * k < nmax) load_scores(sc + (int64_t)min(tid + ST * k, nmax - 1) * GS, G, sv[k]);
  {
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < 16; ++k) M = fmaxf(M, pl + 32 * k < a.W ? pv[k].x : -INFINITY);
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 32));
    float S = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const bool ok = pl + 32 * k < a.W && pv[k].x != -INFINITY;
      S += ok ? pv[k].y * zexp(pv[k].x - M) : 0.0f;
    }
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) S += __shfl_xor(S, o, 32);
    if (pl == 0 && ph < G) sh.lse[ph] = M == -INFINITY ? -INFINITY : M + zlog(S);
    if (tid == 0) { sh.last_kept_id = 0; sh.cut.above = 0; }
    hist_clear(sh.cut);
  }
  __syncthreads();
  float lse[16];
#pragma unroll
  for (int h = 0; h < 16; ++h) lse[h] = h < G ? sh.lse[h] : 0.0f;
  const float invG = 1.0f / (float)G;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  u64 tot = 0;
  for (int b0 = 0; b0 < nmax; b0 += ST * SBATCH) {
#pragma unroll
    for (int k = 0; k < SBATCH; ++k) {
      if (b0 + ST * k < nmax) {
        const int pos = b0 + tid + ST * k;
        const uint32_t key = mass_key(sv[k], lse, G, invG);
        const bool ok = pos < nF;
        if (ok) sh.keys[pos] = key;
        mn = min(mn, ok ? key : 0xFFFFFFFFu);
        mx = max(mx, ok ? key : 0u);
        tot += ok ? fx_mass(key) : 0;
      }
    }
    const int b1 = b0 + ST * SBATCH;
#pragma unroll
    for (int k = 0; k < SBATCH; ++k)
      if (b1 + ST * k < nmax) load_scores(sc + (int64_t)min(b1 + tid + ST * k, nmax - 1) * GS, G, sv[k]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
    tot += __shfl_xor(tot, o);
  }
  if (lane == 0) { sh.mn[wave] = mn; sh.mx[wave] = mx; sh.cut.red64[wave] = tot; }
  __syncthreads();
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  u64 total = 0;
#pragma unroll
  for (int w = 0; w < ST / 64; ++w) {
    kmin = min(kmin, sh.mn[w]);
    kmax = max(kmax, sh.mx[w]);
    total += sh.cut.red64[w];
  }
  uint32_t tau = 0;
  int tie_last = 0x7FFFFFFF;
  const bool keep_all = a.keep_all || nF == 0 || total == 0;  // total 0: every mass rounds to zero
  if (!keep_all) {
    const u64 T = target_of(a.p, total);
    __syncthreads();
    hist_keys_lds(sh.cut, sh.keys, nF, kmin, kmax);
    __syncthreads();
    resolve_cut_lds(sh.cut, sh.keys, nullptr, nF, kmin, kmax, T, nullptr, 0, 0, &tau, &tie_last);
  }
  // compaction in position order (chunks of 4 positions per thread)
  int32_t* kept = a.kept + (int64_t)u * a.capl;
  u64* kr = a.krank ? a.krank + (int64_t)u * a.capl : nullptr;
  uint32_t* uf = a.uflag ? a.uflag + (int64_t)union_group(u, a.hr, a.Hkv, a.Tq, a.TS, a.NTC) * a.ufstride : nullptr;
  const int32_t* par = gpar ? sh.par : nullptr;
  uint32_t kept_base = 0;
  for (int base = 0; base < nF; base += ST * 4) {
    const int p0 = base + tid * 4;
    uint32_t flags = 0, nk = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pos = p0 + e;
      const uint32_t k = sh.keys[min(pos, nF - 1)];
      const bool kp = pos < nF && (keep_all || k > tau || (k == tau && pos <= tie_last));
      flags |= kp ? (1u << e) : 0u;
      nk += kp ? 1u : 0u;
    }
    uint32_t ctot;
    uint32_t out = kept_base + block_excl_scan<ST>(nk, &ctot, sh.cut.scan);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if ((flags >> e) & 1u) {
        const int id = frontier_id(par, p0 + e, a.v.C, a.v.Cshift);
        if (kr) kr[id] = ((u64)stamp << 32) | out;
        if (uf) uf[id] = stamp;
        kept[out++] = id;
        if (p0 + e == nF - 1) sh.last_kept_id = id + 1;  // the frontier's last node is kept
      }
    }
    kept_base += ctot;
  }
  __syncthreads();
  if (tid == 0) {
    a.nF_out[u] = nF;
    a.kept_count[u] = (int)kept_base;
    if (a.next_nF) {
      // every kept node has C children except possibly the level's last node, which can
      // only be the frontier's last position
      const int C = a.v.C;
      int nx = C * (int)kept_base;
      if (sh.last_kept_id > 0) nx = next_frontier((int)kept_base, sh.last_kept_id - 1, C, nchild);
      a.next_nF[u] = nx;
    }
  }
}

// --------------------------------------------------------------------------- large levels

struct MassArgs {
  Level v;
  const float* scores;    // [U][cap1][score row]
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
  // at least 1024 positions per workgroup (one batch of loads per thread): a workgroup's
  // cost is mostly its histogram flush, so a small frontier uses few workgroups
  const int per = max((nF + a.WM - 1) / a.WM, 256 * MASS_BATCH);
  const int start = blockIdx.x * per, end = min(nF, start + per);
  if (start >= end) return;
  const int G = a.G;
  const int GS = score_stride(G);
  const float* sc = a.scores + (int64_t)u * a.cap1 * GS;
  // the first batch of scores is in flight while the frontier's LSE is formed
  float4 sv[MASS_BATCH][4];
#pragma unroll
  for (int k = 0; k < MASS_BATCH; ++k) load_scores(sc + (int64_t)min(start + tid + 256 * k, end - 1) * GS, G, sv[k]);
  frontier_lse256(a.part, a.W, G, u, s_lse);
  for (int i = tid; i < NB; i += 256) { h_cnt[i] = 0; h_mass[i] = 0; }
  __syncthreads();
  uint32_t wlo, whi;
  fine_window(nF, &wlo, &whi);
  const float invG = 1.0f / (float)G;
  uint32_t* keys = a.keys + (int64_t)u * a.kstride;
  u64 am = 0, bm = 0;
  for (int p0 = start + tid; p0 < end; p0 += 256 * MASS_BATCH) {
    if (p0 > start + tid) {
#pragma unroll
      for (int k = 0; k < MASS_BATCH; ++k) load_scores(sc + (int64_t)min(p0 + 256 * k, end - 1) * GS, G, sv[k]);
    }
#pragma unroll
    for (int k = 0; k < MASS_BATCH; ++k) {
      const int pos = p0 + 256 * k;
      if (pos < end) {
        const uint32_t key = mass_key(sv[k], s_lse, G, invG);
        keys[pos] = key;
        if (key > whi) am += fx_mass(key);
        else if (key >= wlo) {
          const uint32_t bn = range_bin(key, wlo, FINE_SHIFT);
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
  uint32_t* cand;         // [U][KSS][LCAND][2]: (key, position) of the crossing slice found by
                          // each workgroup, in any order (written and read with agent-scope atomics)
  uint32_t* ctr;          // [U][1 + KSMAX]: workgroups arrived (zero between launches), then the
                          // number of candidates each workgroup wrote
  int KS;                 // workgroups per unit (<= KSS)
  int KSS;                // candidate regions per unit
  float p;
};

// Resolves the cut of a large frontier with KS workgroups per unit.  The first histogram
// is the fine one built by the mass kernel.  When the cut lies in its window and the
// crossing slice holds at most LCAND keys, every workgroup finds that slice and copies the
// (key, position) pairs of its share of the frontier that fall in it to the unit's
// candidate buffer; the last workgroup to arrive (an acquire-release counter, so it sees
// every other workgroup's candidates) resolves the cut among them in LDS.  Otherwise the
// last workgroup resolves the cut alone over every key.  Output per unit: tau, and the
// position of the last kept key equal to tau (equal keys are taken in position order), so
// that the compaction is a per-position test.
constexpr int LCAND = 8192;  // crossing-slice keys of a large level held in LDS
constexpr int KSMAX = 32;    // selection workgroups per unit at most

// Candidate regions per unit: at most KSMAX, and few enough that every workgroup of a
// launch is resident at once (one per compute unit).
int sel_regions(int U) {
  const int k = 256 / (U > 0 ? U : 1);
  return k < 1 ? 1 : (k > KSMAX ? KSMAX : k);
}
// Workgroups per unit: one per 4096 nodes, at most one per region.
int sel_large_wgs(int64_t cap, int U) {
  const int64_t k = cap / 4096;
  return k < 1 ? 1 : (int)(k < sel_regions(U) ? k : sel_regions(U));
}

__global__ __launch_bounds__(ST) void zha_select_large_kernel(LargeArgs a) {
  __shared__ CutSh sh;
  __shared__ __attribute__((aligned(16))) uint32_t s_ck[LCAND];
  __shared__ __attribute__((aligned(16))) uint32_t s_cp[LCAND];
  __shared__ u64 s_tot[2];
  __shared__ uint32_t s_mn[ST / 64], s_mx[ST / 64];
  __shared__ int s_last;
  __shared__ uint32_t s_wcnt;
  __shared__ uint32_t s_off[KSMAX + 1], s_xoff[KSMAX + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int u = blockIdx.y, j = blockIdx.x;
  uint32_t* ctr = a.ctr + (int64_t)u * (1 + KSMAX);
  const int nF = frontier_size(a.v, u);
  const int kcap = (int)a.kstride;
  const uint32_t* keys = a.keys + (int64_t)u * a.kstride;
  uint32_t* gc = a.fh_cnt + (int64_t)u * NB;
  u64* gm = a.fh_mass + (int64_t)u * NB;
  // every workgroup reads the unit's histogram
#pragma unroll
  for (int e = 0; e < BPT; ++e) {
    sh.hcnt[tid + ST * e] = gc[tid + ST * e];
    sh.hmass[tid + ST * e] = gm[tid + ST * e];
  }
  if (tid < 2) s_tot[tid] = a.fh_edge[u * 2 + tid];
  if (tid == 0) s_wcnt = 0;
  __syncthreads();
  // window mass: workgroup sum of the bins
  u64 wm = sh.hmass[tid] + sh.hmass[tid + ST];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) wm += __shfl_xor(wm, o);
  if (lane == 0) sh.red64[wave] = wm;
  __syncthreads();
  wm = 0;
#pragma unroll
  for (int w = 0; w < ST / 64; ++w) wm += sh.red64[w];
  const u64 above = s_tot[0], total = above + wm + s_tot[1];
  const bool keep_all = nF == 0 || total == 0;  // total 0: every mass rounds to zero
  const u64 T = keep_all ? 0 : target_of(a.p, total);
  const bool inwin = !keep_all && T > above && T <= above + wm;  // the cut lies in the window
  uint32_t wlo = 0, whi = 0, nlo = 0, nhi = 0, cnt = 0;
  bool gathered = false;
  if (inwin) {
    fine_window(nF, &wlo, &whi);
    if (tid == 0) sh.above = above;
    __syncthreads();
    find_bin(sh, T);
    slice_range(wlo, whi, sh.bin, &nlo, &nhi);
    cnt = sh.hcnt[sh.bin];
    gathered = cnt <= (uint32_t)LCAND;  // the same decision in every workgroup
    if (gathered) {
      // this workgroup's share: blocks of 4 * ST positions dealt in turn, four blocks in
      // flight per thread; hits are written from registers to this workgroup's own region,
      // one LDS reservation per wave
      u64* cand = (u64*)a.cand + ((int64_t)u * a.KSS + j) * LCAND;  // key low, position high
      for (int b0 = j; b0 * 4 * ST < nF; b0 += 4 * a.KS) {
        uint4 kv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) kv[r] = load4c(keys, ((b0 + r * a.KS) * ST + tid) * 4, kcap);
        uint32_t mask = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int p0 = ((b0 + r * a.KS) * ST + tid) * 4;
          const uint32_t k4[4] = {kv[r].x, kv[r].y, kv[r].z, kv[r].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool hit = p0 + e < nF && k4[e] >= nlo && k4[e] <= nhi;
            mask |= hit ? 1u << (4 * r + e) : 0u;
          }
        }
        const uint32_t c = (uint32_t)__popc(mask);
        uint32_t inc = c;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t y = __shfl_up(inc, o);
          if (lane >= o) inc += y;
        }
        uint32_t wbase = 0;
        if (lane == 63 && inc) wbase = atomicAdd(&s_wcnt, inc);
        wbase = __shfl(wbase, 63);
        uint32_t slot = wbase + inc - c;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int p0 = ((b0 + r * a.KS) * ST + tid) * 4;
          const uint32_t k4[4] = {kv[r].x, kv[r].y, kv[r].z, kv[r].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if ((mask >> (4 * r + e)) & 1u) {
              if (slot < (uint32_t)LCAND)
                __hip_atomic_store(&cand[slot], ((u64)(uint32_t)(p0 + e) << 32) | k4[e], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
              ++slot;
            }
          }
        }
      }
    }
  }
  // arrive; the last workgroup of the unit goes on
  __syncthreads();
  if (tid == 0) {
    __hip_atomic_store(&ctr[1 + j], s_wcnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t before = __hip_atomic_fetch_add(&ctr[0], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_last = before == (uint32_t)(a.KS - 1) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;
  // every workgroup has read the histogram and written its candidates
  uint32_t tau = 0;
  int tie_last = 0x7FFFFFFF;
  if (!keep_all) {
    if (gathered) {
      // The workgroups' regions, concatenated.  The counts and the first E0 entries of every
      // region are loaded together (entries past a region's count are ignored), then the
      // rare remainder of longer regions.
      const u64* cand = (const u64*)a.cand + (int64_t)u * a.KSS * LCAND;
      const int E0 = ST / a.KS;
      const int w0 = tid / E0, k0 = tid - w0 * E0;
      const bool own = w0 < a.KS;
      const u64 c0 = own ? __hip_atomic_load(&cand[(int64_t)w0 * LCAND + k0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                         : 0;
      if (wave == 0) {  // exclusive scans of the KS <= 32 counts and of their excess over E0
        const uint32_t cw = lane < a.KS ? __hip_atomic_load(&ctr[1 + lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                        : 0u;
        const uint32_t xw = cw > (uint32_t)E0 ? cw - (uint32_t)E0 : 0u;
        uint32_t inc = cw, xinc = xw;
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) {
          const uint32_t y = __shfl_up(inc, o), xy = __shfl_up(xinc, o);
          if (lane >= o) { inc += y; xinc += xy; }
        }
        if (lane < a.KS) { s_off[lane] = inc - cw; s_xoff[lane] = xinc - xw; }
        if (lane == a.KS - 1) { s_off[a.KS] = inc; s_xoff[a.KS] = xinc; }
      }
      __syncthreads();
      if (own && (uint32_t)k0 < s_off[w0 + 1] - s_off[w0]) {
        s_ck[s_off[w0] + k0] = (uint32_t)c0;
        s_cp[s_off[w0] + k0] = (uint32_t)(c0 >> 32);
      }
      // entries past the first E0 of their region, all loads of a pass issued together
      const int X = (int)s_xoff[a.KS];
      for (int x = tid; x < X; x += ST) {
        int lo = 0, hi = a.KS - 1;  // the region w with s_xoff[w] <= x < s_xoff[w + 1]
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (s_xoff[mid] <= (uint32_t)x) lo = mid; else hi = mid - 1;
        }
        const int k = E0 + (x - (int)s_xoff[lo]);
        const u64 c = __hip_atomic_load(&cand[(int64_t)lo * LCAND + k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_ck[s_off[lo] + k] = (uint32_t)c;
        s_cp[s_off[lo] + k] = (uint32_t)(c >> 32);
      }
      __syncthreads();
      if (cnt <= (uint32_t)RMAX) {
        if (tid < (int)cnt) {
          sh.rkey[tid] = s_ck[tid];
          sh.rpos[tid] = s_cp[tid];
        }
        __syncthreads();
        rank_cut(sh, (int)cnt, T);
        tau = sh.tau;
        tie_last = sh.tie_last;
      } else {
        hist_clear(sh);
        __syncthreads();
        hist_keys_lds(sh, s_ck, (int)cnt, nlo, nhi);
        __syncthreads();
        resolve_cut_lds(sh, s_ck, s_cp, (int)cnt, nlo, nhi, T, keys, nF, kcap, &tau, &tie_last);
      }
    } else {
      uint32_t lo, hi;
      if (inwin) {  // crossing slice of more than LCAND keys: start again from the fine histogram
        lo = wlo;
        hi = whi;
        if (tid == 0) sh.above = above;
      } else {
        // every key over its whole range
        uint32_t mn = 0xFFFFFFFFu, mx = 0u;
        for (int base = 4 * tid; base < nF; base += 4 * ST) {
          const uint4 kv = load4c(keys, base, kcap);
          const uint32_t k4[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (base + e < nF) { mn = min(mn, k4[e]); mx = max(mx, k4[e]); }
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
          mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
          mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
        }
        if (lane == 0) { s_mn[wave] = mn; s_mx[wave] = mx; }
        hist_clear(sh);
        if (tid == 0) sh.above = 0;
        __syncthreads();
        lo = 0xFFFFFFFFu;
        hi = 0u;
#pragma unroll
        for (int w = 0; w < ST / 64; ++w) { lo = min(lo, s_mn[w]); hi = max(hi, s_mx[w]); }
        hist_keys(sh, keys, nF, kcap, lo, hi);
      }
      __syncthreads();
      resolve_cut(sh, keys, nF, kcap, lo, hi, T, s_ck, s_cp, LCAND, &tau, &tie_last);
    }
  }
  if (tid == 0) {
    a.cut[u * 4 + 0] = (int32_t)tau;
    a.cut[u * 4 + 1] = tie_last;
    a.cut[u * 4 + 2] = keep_all ? 1 : 0;
  }
  // leave the unit's histogram and counters at zero for the next level (last, so that no
  // workgroup barrier waits for these stores)
#pragma unroll
  for (int e = 0; e < BPT; ++e) {
    gc[tid + ST * e] = 0;
    gm[tid + ST * e] = 0;
  }
  if (tid < 2) a.fh_edge[u * 2 + tid] = 0;
  if (tid == 0) ctr[0] = 0;
}

struct CompactArgs {
  Level v;
  const uint32_t* keys;   // [U][kstride]
  int64_t kstride;
  const int32_t* cut;     // [U][4]
  int keep_all;           // p >= 1: every position is kept (cut unused)
  u64* status;            // [U][nchunk] look-back words
  int nchunk;
  uint32_t* epoch;        // [U][2]: epoch of the unit's status words (starts at 1), its finished workgroups
  int32_t* kept;          // [U][capl]
  int64_t capl;
  int32_t* nF_out;
  int32_t* kept_count;
  int32_t* next_nF;       // null at level 1
  int32_t* lb_error;      // set when a look-back wait gives up (never expected)
  u64* krank;             // union routes: [U][capl] (stamp << 32) | rank of each kept node; else null
  const uint32_t* route_ctr;  // the route's stamp
  uint32_t* uflag;        // union routes at level 1: [groups][kstride] stamp of every kept chunk
  int hr, Hkv, Tq, TS, NTC;  // routing-unit numbering and union groups (for the unit's group)
  int stamp_keys;         // 1: keep the positions whose key equals the route's stamp (no cut)
};

constexpr int CPT = 256;  // compaction threads
constexpr int CPP = 16;   // positions per thread (contiguous)
static_assert(CH == CPT * CPP, "compaction chunk");

__device__ __forceinline__ u64 lb_word(uint32_t epoch, int inclusive, uint32_t count) {
  return ((u64)epoch << 32) | ((u64)inclusive << 31) | (u64)count;
}

__device__ __forceinline__ void compact_epilogue(const CompactArgs& a) {
  // the last workgroup of the unit advances the unit's epoch: every workgroup of the unit
  // read it before finishing (one counter per unit keeps the atomics on one address few)
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t* ep = a.epoch + 2 * blockIdx.y;
    if (atomicAdd(&ep[1], 1u) == gridDim.x - 1) {
      __hip_atomic_store(&ep[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t e = __hip_atomic_load(&ep[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&ep[0], e + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Kept count of the chunks before chunk c (c >= 1), by a decoupled look-back run by one
// wave: lane l reads the status word of chunk c-1-l, all 64 at once, waiting (bounded) on
// words not yet published in this epoch; the nearest inclusive word ends the walk, else
// the window moves 64 chunks back.
__device__ __forceinline__ uint32_t look_back(const u64* st, int c, uint32_t epoch, int32_t* lb_error) {
  const int lane = threadIdx.x & 63;
  uint32_t before = 0;
  for (int top = c - 1; top >= 0; top -= 64) {
    const int j = top - lane;
    u64 w = lb_word(epoch, 1, 0);  // past chunk 0: nothing more to add
    if (j >= 0) {
      int spins = 0;
      for (;;) {
        w = __hip_atomic_load(&st[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((uint32_t)(w >> 32) == epoch) break;
        if (++spins > (1 << 22)) {  // bounded wait: flag and continue rather than hang
          atomicExch(lb_error, 1);
          w = lb_word(epoch, 1, 0);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    const bool incl = ((w >> 31) & 1u) != 0;
    const u64 mask = __ballot(incl);
    const int first = mask ? __ffsll((unsigned long long)mask) - 1 : 64;
    uint32_t v = lane <= first ? (uint32_t)(w & 0x7FFFFFFFu) : 0u;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    before += v;
    if (mask) break;
  }
  return before;
}

// Writes the kept ids of one chunk of CH positions, in order.  Position i is kept when its
// key is above the cut, or equals it and i is not after the last kept tie.  The kept
// counts of earlier chunks arrive by the look-back (chunk c waits only on chunks < c,
// which are dispatched before it).  The chunk holding the frontier's last position writes
// the level's counts.
__global__ __launch_bounds__(CPT) void zha_compact_kernel(CompactArgs a) {
  __shared__ uint32_t s_scan[CPT / 64];
  __shared__ uint32_t s_before, s_epoch;
  __shared__ int s_last_kept;
  const int tid = threadIdx.x;
  const int u = blockIdx.y, c = blockIdx.x;
  const int nF = frontier_size(a.v, u);
  const int base = c * CH;
  const int nchild = a.next_nF && base + CH >= nF ? child_nodes(a.v, u) : 0;  // loaded now, used at the end
  if (tid == 0) s_epoch = __hip_atomic_load(&a.epoch[2 * u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (base >= nF) {
    if (c == 0 && tid == 0) {  // an empty frontier (a sequence without nodes at this level)
      a.nF_out[u] = 0;
      a.kept_count[u] = 0;
      if (a.next_nF) a.next_nF[u] = 0;
    }
    compact_epilogue(a);
    return;
  }
  const uint32_t stamp = (a.krank || a.uflag || a.stamp_keys) ? a.route_ctr[0] : 0u;
  const bool keep_all = !a.stamp_keys && (a.keep_all || a.cut[u * 4 + 2] != 0);
  const uint32_t tau = a.stamp_keys ? 0u : (uint32_t)a.cut[u * 4 + 0];
  const int tie_last = a.stamp_keys ? 0 : a.cut[u * 4 + 1];
  const uint32_t* keys = a.keys + (int64_t)u * a.kstride;
  const int32_t* par = a.v.parent ? a.v.parent + (int64_t)u * a.v.cap_parent : nullptr;
  const int p0 = base + CPP * tid;
  uint4 kv[CPP / 4];
#pragma unroll
  for (int j = 0; j < CPP / 4; ++j) kv[j] = load4c(keys, p0 + 4 * j, (int)a.kstride);
  // node ids of the positions (independent of the prefix: loaded before the look-back)
  int id[CPP];
#pragma unroll
  for (int e = 0; e < CPP; ++e) id[e] = frontier_id(par, min(p0 + e, nF - 1), a.v.C, a.v.Cshift);
  uint32_t flags = 0;
#pragma unroll
  for (int j = 0; j < CPP / 4; ++j) {
    const uint32_t k4[4] = {kv[j].x, kv[j].y, kv[j].z, kv[j].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pos = p0 + 4 * j + e;
      const bool kp = pos < nF && (a.stamp_keys ? k4[e] == stamp
                                                 : (keep_all || k4[e] > tau || (k4[e] == tau && pos <= tie_last)));
      flags |= kp ? (1u << (4 * j + e)) : 0u;
    }
  }
  uint32_t tot;
  const uint32_t ex = block_excl_scan<CPT>((uint32_t)__popc(flags), &tot, s_scan);
  u64* st = a.status + (int64_t)u * a.nchunk;
  const uint32_t epoch = s_epoch;
  if (tid == 0)
    __hip_atomic_store(&st[c], lb_word(epoch, c == 0 ? 1 : 0, tot), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (c > 0 && tid < 64) {
    const uint32_t before = look_back(st, c, epoch, a.lb_error);
    if (tid == 0) {
      __hip_atomic_store(&st[c], lb_word(epoch, 1, before + tot), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_before = before;
    }
  } else if (tid == 0) {
    s_before = 0;
  }
  if (tid == 0) s_last_kept = 0;
  __syncthreads();
  uint32_t out = s_before + ex;
  int32_t* kept = a.kept + (int64_t)u * a.capl;
  u64* kr = a.krank ? a.krank + (int64_t)u * a.capl : nullptr;
  uint32_t* uf = a.uflag ? a.uflag + (int64_t)union_group(u, a.hr, a.Hkv, a.Tq, a.TS, a.NTC) * a.kstride : nullptr;
#pragma unroll
  for (int e = 0; e < CPP; ++e) {
    if ((flags >> e) & 1u) {
      if (kr) kr[id[e]] = ((u64)stamp << 32) | out;
      if (uf) uf[id[e]] = stamp;
      kept[out++] = id[e];
      if (p0 + e == nF - 1) s_last_kept = id[e] + 1;  // the frontier's last node is kept
    }
  }
  __syncthreads();
  if (base + CH >= nF && tid == 0) {
    const uint32_t total = s_before + tot;
    a.nF_out[u] = nF;
    a.kept_count[u] = (int)total;
    if (a.next_nF) {
      // every kept node has C children except possibly the level's last node, which can
      // only be the frontier's last position
      const int C = a.v.C;
      int nx = C * (int)total;
      if (s_last_kept > 0) nx = next_frontier((int)total, s_last_kept - 1, C, nchild);
      a.next_nF[u] = nx;
    }
  }
  compact_epilogue(a);
}

// Two tiles per wave per pipeline stage (for fp8 codes too: four would not fit in the
// registers of four workgroups per compute unit, and fewer workgroups measured slower; for
// fp4 codes four or eight tiles measured slower too).
// SM: summary storage (0 native, 1 fp8, 2 fp4)
template <typename T, int R, int D, int SM, bool UNI, int NT = 1, bool PSEL = false>
hipError_t launch_score(const ScoreArgs& a, int W, int rows, hipStream_t s) {
  if constexpr (!UNI && !PSEL) {  // the streaming levels of one-unit rows: shifts for power-of-two chunks
    if (a.v.Cshift >= 0) {
      hipLaunchKernelGGL((zha_score_kernel<T, R, D, 2, SM, false, 1, false, true>), dim3(W, rows), dim3(256), 0, s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((zha_score_kernel<T, R, D, 2, SM, UNI, NT, PSEL>), dim3(W, rows), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int R, int D, int SM>
hipError_t launch_score_uni(const ScoreArgs& a, int W, int rows, int NT, hipStream_t s) {
  switch (NT) {
    case 1: return launch_score<T, R, D, SM, true, 1>(a, W, rows, s);
    case 2: return launch_score<T, R, D, SM, true, 2>(a, W, rows, s);
    default: return launch_score<T, R, D, SM, true, 4>(a, W, rows, s);
  }
}

// rows: routing units, or groups of them (uni; R >= 4 there, NT column tiles of 16); psel:
// the parent level's selection runs in every workgroup (one routing unit per row)
template <typename T, int D, int SM = 0>
hipError_t launch_score_r(const ScoreArgs& a, int R, int W, int rows, bool uni, int NT, bool psel, hipStream_t s) {
  if (psel) {
    switch (R) {
      case 1: return launch_score<T, 1, D, SM, false, 1, true>(a, W, rows, s);
      case 2: return launch_score<T, 2, D, SM, false, 1, true>(a, W, rows, s);
      case 4: return launch_score<T, 4, D, SM, false, 1, true>(a, W, rows, s);
      case 8: return launch_score<T, 8, D, SM, false, 1, true>(a, W, rows, s);
      default: return launch_score<T, 16, D, SM, false, 1, true>(a, W, rows, s);
    }
  }
  if (uni) {
    switch (R) {
      case 4: return launch_score_uni<T, 4, D, SM>(a, W, rows, NT, s);
      case 8: return launch_score_uni<T, 8, D, SM>(a, W, rows, NT, s);
      default: return launch_score_uni<T, 16, D, SM>(a, W, rows, NT, s);
    }
  }
  switch (R) {
    case 1: return launch_score<T, 1, D, SM, false>(a, W, rows, s);
    case 2: return launch_score<T, 2, D, SM, false>(a, W, rows, s);
    case 4: return launch_score<T, 4, D, SM, false>(a, W, rows, s);
    case 8: return launch_score<T, 8, D, SM, false>(a, W, rows, s);
    default: return launch_score<T, 16, D, SM, false>(a, W, rows, s);
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
int zha_score_wgs_units(int RU) {
  int ws = 2048 / (RU > 0 ? RU : 1);  // two rounds of four workgroups per compute unit in all
  if (ws > 512) ws = 512;
  return ws < 1 ? 1 : ws;
}

int zha_score_wgs(const zha_tree* t, int level) {
  const int per = 8;  // nodes of one super-tile at R = 16
  int64_t w = (t->cap[level] + per - 1) / per;
  if (w < 1) w = 1;
  if (w > t->WS) w = t->WS;
  return (int)w;
}

// Union groups hold the routing units that share one (sequence, KV head): the hr units of
// each of TS consecutive queries.  Scoring groups up to 64 query heads (four column tiles in
// every wave, one plane load for all of them).  Attention (and the kept-chunk flags the
// selections write for it) groups up to 64 with bf16 K/V (windows staged once in LDS for
// the workgroup's waves, one column tile per wave) and up to 16 otherwise (one column
// tile).  Only worth it (and only built) when a group holds several units and a tile row
// holds one node's planes for one lane group (R >= 4).
static int union_queries(int R, int Gq, int Tq, int hr, int cols) {
  if (R < 4 || Gq < 1 || Gq > 16) return 0;
  int ts = cols / Gq;
  if (ts > Tq) ts = Tq;
  if (ts < 1) ts = 1;
  return ts * hr > 1 ? ts : 0;
}
int zha_union_queries(int R, int Gq, int Tq, int hr, bool wide) { return union_queries(R, Gq, Tq, hr, wide ? 64 : 16); }
int zha_union_score_queries(int R, int Gq, int Tq, int hr) { return union_queries(R, Gq, Tq, hr, 64); }

int zha_compact_chunks(int64_t nodes) { return (int)((nodes + CH - 1) / CH); }
int zha_small_score_rows() { return WN; }  // rows per routing unit of the small score buffers
int zha_hist_bins() { return NB; }
int64_t zha_sel_cand_entries(int U) { return (int64_t)U * sel_regions(U) * LCAND; }
int zha_sel_ctr_words(int U) { return U * (1 + KSMAX); }

hipError_t zha_launch_route(zha_tree* t, const void* q, float p, float scale, hipStream_t s) {
  // U: routing units of this route (t->U * Tq (sequence, query, KV head) triples, times G
  // (one per query head) for per-head routes); Gr: query heads per routing unit
  const int U = t->RU, L = t->L, Gr = t->G / t->hr;
  const int Cshift = cshift_of(t->C);
  int32_t* cntF = t->counts;                         // [L+2][U]
  int32_t* cntK = t->counts + (int64_t)(L + 2) * U;  // [L+2][U]
  const bool keep_all = p >= 1.0f;
  // union scoring: groups of the units sharing one (sequence, KV head), TS queries each
  // Union kernels pay a walk over each level's node ids (scoring), or a list per group and
  // every listed token computed for every column (attention).  Scoring wins when the units'
  // kept sets overlap much (high p) or a group holds many units; attention only when they
  // overlap much: high p, or the heads of one query (measured: a block of 8 queries at
  // p = 0.7, batch 8, attends 2.7x slower over the union than per unit).
  const int TS = zha_union_queries(t->R, t->G, t->Tq, t->hr, t->desc.dtype == ZHA_BF16);  // attention groups
  const int TSs = zha_union_score_queries(t->R, t->G, t->Tq, t->hr);  // scoring groups
  const bool can = t->krank[1] != nullptr;
  const bool uni = can && TS > 0 && (p >= 0.8f || (t->hr >= 4 && t->Tq == 1));
  const bool uni_s = can && TSs > 0 && (TSs * t->hr >= 4 || p >= 0.8f);
  t->uni_route = uni;
  const int NTC = uni ? (t->Tq + TS - 1) / TS : 1;
  const int NTCs = uni_s ? (t->Tq + TSs - 1) / TSs : 1;
  const int NT = uni_s ? (TSs * t->G + 15) / 16 : 1;  // column tiles of a scoring group
  const int rows = uni_s ? t->U * NTCs : U;             // rows of the scoring grid
  hipError_t e;
  // Scores and scoring partials of consecutive levels live in different buffers, so a launch
  // can read one level's while writing the next's: a level of at most WN nodes writes the
  // small score buffer of its parity, a larger one the full buffer; partials alternate by
  // parity.
  auto sbuf = [&](int l) { return t->cap[l] <= WN ? t->sscore[l & 1] : t->scores; };
  auto sstride = [&](int l) { return t->cap[l] <= WN ? (int64_t)WN : t->cap[1]; };
  auto pbuf = [&](int l) { return t->spart[l & 1]; };
  // Levels of at most WN nodes in routes of one-unit rows are selected by the next level's
  // scoring launch (every workgroup selects them itself, from their scores and partials).
  auto deferred = [&](int l) { return !uni_s && l > 1 && t->cap[l] <= WN; };
  Level pvl;  // the previous (parent) level, for the next launch's selection of it
  for (int l = L; l >= 1; --l) {
    Level v;
    v.parent = l < L ? t->kept[l + 1] : nullptr;
    v.parent_nF = l < L ? cntF + (int64_t)l * U : nullptr;  // written by level l+1
    v.cap_parent = l < L ? t->cap[l + 1] : 0;
    v.C = t->C;
    v.Cshift = Cshift;
    v.Hkv = t->desc.n_kv_heads * t->hr * t->Tq;  // routing units per sequence
    v.nodes = t->geo + (int64_t)l * t->desc.batch;
    v.child = t->geo + (int64_t)(l - 1) * t->desc.batch;
    int32_t* next_nF = l > 1 ? cntF + (int64_t)(l - 1) * U : nullptr;

    ScoreArgs sa;
    sa.v = v;
    sa.m = t->m[l];
    sa.b = t->b[l];
    sa.ms = t->ms[l];
    sa.q = q;
    sa.capl = t->cap[l];
    sa.scores = sbuf(l);
    sa.cap1 = sstride(l);
    sa.part = pbuf(l);
    const bool psel = l < L && deferred(l + 1);
    if (psel) {
      sa.pv = pvl;
      sa.pscores = sbuf(l + 1);
      sa.pstride = sstride(l + 1);
      sa.pkept = t->kept[l + 1];
      sa.pcapl = t->cap[l + 1];
      sa.pnF_out = cntF + (int64_t)(l + 1) * U;
      sa.pkept_count = cntK + (int64_t)(l + 1) * U;
      sa.nF_out = cntF + (int64_t)l * U;
    }
    sa.p = p;
    sa.keep_all = keep_all ? 1 : 0;
    if (uni_s) {
      int64_t w = (t->cap[l] + 7) / 8;
      const int wr = zha_score_wgs_units(rows);
      sa.W = (int)(w < 1 ? 1 : (w > wr ? wr : w));
    } else {
      sa.W = zha_score_wgs(t, l);
      // every workgroup of a launch that selects the parent level pays for that selection:
      // one round of resident workgroups (three per compute unit) pays it once
      if (psel) sa.W = std::max(1, std::min(sa.W, 768 / U));
    }
    sa.krank = uni_s && l < L ? t->krank[l + 1] : nullptr;
    sa.route_ctr = (uni || uni_s) ? t->route_ctr : nullptr;
    sa.TS = TSs;
    sa.NTC = NTCs;
    sa.G = Gr;
    sa.hr = t->hr;
    sa.Hkv = t->desc.n_kv_heads;
    sa.Tq = t->Tq;
    sa.scale = scale;
    zha_time_begin(t, s, ZHA_K_SCORE, l);
    if (t->f8)
      e = t->d == 64 ? launch_score_r<__bf16, 64, 1>(sa, t->R, sa.W, rows, uni_s, NT, psel, s)
                     : launch_score_r<__bf16, 128, 1>(sa, t->R, sa.W, rows, uni_s, NT, psel, s);
    else if (t->f4)
      e = t->d == 64 ? launch_score_r<__bf16, 64, 2>(sa, t->R, sa.W, rows, uni_s, NT, psel, s)
                     : launch_score_r<__bf16, 128, 2>(sa, t->R, sa.W, rows, uni_s, NT, psel, s);
    else if (t->desc.dtype == ZHA_BF16)
      e = t->d == 64 ? launch_score_r<__bf16, 64>(sa, t->R, sa.W, rows, uni_s, NT, psel, s)
                     : launch_score_r<__bf16, 128>(sa, t->R, sa.W, rows, uni_s, NT, psel, s);
    else
      e = t->d == 64 ? launch_score_r<float, 64>(sa, t->R, sa.W, rows, uni_s, NT, psel, s)
                     : launch_score_r<float, 128>(sa, t->R, sa.W, rows, uni_s, NT, psel, s);
    if (e != hipSuccess) return e;
    zha_time_end(t, s, ZHA_K_SCORE, l);
    pvl = v;
    if (deferred(l)) continue;  // selected by the next level's scoring launch

    if (!uni_s && t->cap[l] <= WN) {
      WaveArgs wa;
      wa.v = v;
      wa.scores = sbuf(l);
      wa.sstride = sstride(l);
      wa.G = Gr;
      wa.p = p;
      wa.keep_all = keep_all ? 1 : 0;
      wa.kept = t->kept[l];
      wa.capl = t->cap[l];
      wa.nF_out = cntF + (int64_t)l * U;
      wa.kept_count = cntK + (int64_t)l * U;
      wa.next_nF = next_nF;
      zha_time_begin(t, s, ZHA_K_SELECT, l);
      hipLaunchKernelGGL(zha_select_wave_kernel, dim3(U), dim3(SSEL), 0, s, wa);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      zha_time_end(t, s, ZHA_K_SELECT, l);
      continue;
    }
    if (t->cap[l] <= SMALL_NODES) {
      SmallArgs sm;
      sm.v = v;
      sm.scores = sbuf(l);
      sm.cap1 = sstride(l);
      sm.part = pbuf(l);
      sm.W = sa.W;
      sm.kept = t->kept[l];
      sm.capl = t->cap[l];
      sm.npar = (int)((t->cap[l] + t->C - 1) / t->C);
      sm.nF_out = cntF + (int64_t)l * U;
      sm.kept_count = cntK + (int64_t)l * U;
      sm.next_nF = next_nF;
      sm.G = Gr;
      sm.p = p;
      sm.keep_all = keep_all ? 1 : 0;
      sm.krank = (uni_s && l > 1) || (uni && l == 1) ? t->krank[l] : nullptr;
      sm.route_ctr = t->route_ctr;
      sm.uflag = uni && l == 1 ? t->uflag : nullptr;
      sm.ufstride = t->kstride;
      sm.hr = t->hr;
      sm.Hkv = t->desc.n_kv_heads;
      sm.Tq = t->Tq;
      sm.TS = TS;
      sm.NTC = NTC;
      zha_time_begin(t, s, ZHA_K_SELECT, l);
      hipLaunchKernelGGL(zha_select_small_kernel, dim3(U), dim3(ST), 0, s, sm);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      zha_time_end(t, s, ZHA_K_SELECT, l);
      continue;
    }
    if (!keep_all) {
      MassArgs ma;
      ma.v = v;
      ma.scores = sbuf(l);
      ma.cap1 = sstride(l);
      ma.part = pbuf(l);
      ma.W = sa.W;
      ma.keys = t->keys;
      ma.kstride = t->kstride;
      ma.fh_cnt = t->fh_cnt;
      ma.fh_mass = (u64*)t->fh_mass;
      ma.fh_edge = (u64*)t->fh_edge;
      ma.G = Gr;
      // 1024 positions per workgroup, at most 512 workgroups in all: every workgroup adds its
      // histogram to the unit's with global atomics, and with many routing units (per-head
      // routes, batches) more workgroups only contend on those addresses
      int64_t wm = (t->cap[l] + 1023) / 1024;
      wm = std::min<int64_t>(wm, std::max(1, 512 / U));
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
      la.cand = t->sel_cand;
      la.ctr = t->sel_ctr;
      la.KS = sel_large_wgs(t->cap[l], U);
      la.KSS = sel_regions(U);
      la.p = p;
      zha_time_begin(t, s, ZHA_K_SELECT, l);
      hipLaunchKernelGGL(zha_select_large_kernel, dim3(la.KS, U), dim3(ST), 0, s, la);
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
    ca.kept = t->kept[l];
    ca.capl = t->cap[l];
    ca.nF_out = cntF + (int64_t)l * U;
    ca.kept_count = cntK + (int64_t)l * U;
    ca.next_nF = next_nF;
    ca.lb_error = t->lb_error;
    ca.krank = (uni_s && l > 1) || (uni && l == 1) ? t->krank[l] : nullptr;
    ca.route_ctr = t->route_ctr;
    ca.uflag = uni && l == 1 ? t->uflag : nullptr;
    ca.hr = t->hr;
    ca.Hkv = t->desc.n_kv_heads;
    ca.Tq = t->Tq;
    ca.TS = TS;
    ca.NTC = NTC;
    ca.stamp_keys = 0;
    const int nch = zha_compact_chunks(t->cap[l]);
    zha_time_begin(t, s, ZHA_K_COMPACT, l);
    hipLaunchKernelGGL(zha_compact_kernel, dim3(nch, U), dim3(CPT), 0, s, ca);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    zha_time_end(t, s, ZHA_K_COMPACT, l);
  }
  if (uni) {
    // the level-1 kept list of every union group: the chunks whose flag holds this route's
    // stamp, in order (what union attention reads); groups are numbered (sequence, KV head,
    // query chunk)
    CompactArgs ca;
    ca.v.parent = nullptr;
    ca.v.parent_nF = nullptr;
    ca.v.cap_parent = 0;
    ca.v.C = t->C;
    ca.v.Cshift = Cshift;
    ca.v.Hkv = t->desc.n_kv_heads * NTC;  // groups per sequence
    ca.v.nodes = t->geo + t->desc.batch;  // level-1 nodes per sequence
    ca.v.child = t->geo;
    ca.keys = t->uflag;
    ca.kstride = t->kstride;
    ca.cut = t->cut;
    ca.keep_all = 0;
    ca.status = (u64*)t->lb_status;
    ca.nchunk = zha_compact_chunks(t->cap[1]);
    ca.epoch = t->lb_epoch;
    ca.kept = t->ulist;
    ca.capl = t->cap[1];
    ca.nF_out = t->ucount + t->U * NTC;
    ca.kept_count = t->ucount;
    ca.next_nF = nullptr;
    ca.lb_error = t->lb_error;
    ca.krank = nullptr;
    ca.route_ctr = t->route_ctr;
    ca.uflag = nullptr;
    ca.hr = 1;
    ca.Hkv = t->desc.n_kv_heads;
    ca.Tq = 1;
    ca.TS = 1;
    ca.NTC = 1;
    ca.stamp_keys = 1;
    zha_time_begin(t, s, ZHA_K_COMPACT, 0);
    hipLaunchKernelGGL(zha_compact_kernel, dim3(zha_compact_chunks(t->cap[1]), t->U * NTC), dim3(CPT), 0, s, ca);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    zha_time_end(t, s, ZHA_K_COMPACT, 0);
  }
  return hipSuccess;
}
