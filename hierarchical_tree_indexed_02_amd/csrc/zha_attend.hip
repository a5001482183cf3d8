// zha_attend.hip -- exact attention over the routed token set, and dense decode.
//
// S = {token 0} U (tokens of the kept leaf chunks) U [Nc, N): the first token is
// always kept as an attention sink, the trailing partial chunk is not in the
// tree and is always read ([wqu] "How does top-p routing pick tokens?"), and
// attention over S is exact softmax attention on the raw, unmodified K/V
// ([wqu] "What is Zyphra Hierarchical Attention (ZHA)?").  Dense decode is the
// same computation with S = [0, N).
//
// Split-K flash decode: the unit's position list (sink and tail first, then the kept
// chunks' tokens in order) is cut into blocks of 128 positions dealt to the workgroups
// in turn; a workgroup's four waves take 32 positions each with an online softmax, and the
// G query heads of the KV head share every K/V tile.  Q.K^T runs on the matrix
// cores with K rows loaded straight from HBM into the operand registers; P.V
// stages the V tile in LDS and reads it transposed.  K and V are read once per step:
// their loads carry the nontemporal hint so they do not displace reused data in the caches.  P is split into two bf16
// halves (hi + lo) so the softmax weights keep ~16 significant bits.  Partial
// (max, sum, o) per workgroup are merged by zha_merge_kernel in fixed order.
//
// Union attention (UNI): the routing units of a group share one KV head (the heads of a
// per-head route, or the queries of a block); the group walks the union of their kept
// chunks once, one matrix column per unit head, and each column's softmax takes only the
// tokens of its own unit's set.
#include "zha_internal.h"

#include <type_traits>

namespace {

struct AttArgs {
  const void* q;           // [B][Tq][Hq][d]
  const void* K;           // [B][Hkv][T][d]
  const void* V;
  const int32_t* kept;     // [U][cap1] level-1 kept chunk ids (sparse only)
  const int32_t* kept_count;
  int64_t cap1;
  float* part;             // o [U][W][G][d] (unnormalised), then (max in log2 units, sum) [U][W][G][2]
  int W, U;                // workgroups per unit; routing units (U = B * Tq * Hkv * hr)
  int hr;                  // routing units per (query, KV head): 1, or G when each head is routed alone
  int Tq;                  // queries per sequence
  int qtail;               // 1: query t of a block also reads the block's rows [N, N + t]
  int Hkv, Hq, G, C, Cshift;
  int64_t T;               // token stride of K/V
  float scale_log2;        // scale * log2(e)
  const int32_t* lens;     // sparse: sequence lengths [B] on the device (the tree's geometry row 0)
  // Union attention: one row of workgroups per group of routing units sharing one (sequence,
  // KV head) (the hr units of TS consecutive queries, at most 16 query heads in all).  The
  // group's tokens are read once, in order, and each query head's softmax takes the tokens
  // of its unit's set only.
  const u64* krank;        // level-1 kept ranks [U][cap1]: (stamp << 32) | rank, by chunk id
  const uint32_t* route_ctr;  // the last route's stamp
  const int32_t* ulist;    // [groups][cap1] chunks kept by some routing unit of the group
  const int32_t* ucount;   // [groups]
  int TS, NTC;             // queries per group; groups per (sequence, KV head)
};

// Dense launches take the lengths by value (the dense entry point gets them from the host);
// sparse launches read them from the tree, so their arguments stay small.
template <bool DENSE> struct LensArg { ZLens len; };
template <> struct LensArg<false> {};

struct Positions {
  int P;        // number of positions
  int nx;       // positions before the chunk tokens (sink, then tail)
  int sink;     // 1 when token 0 is read as a separate sink position
  int Nc;
  int nK;       // kept chunks
  const int32_t* kp;
};

template <bool DENSE>
__device__ __forceinline__ Positions unit_positions(const AttArgs& a, const LensArg<DENSE>& la, int u, int bi) {
  Positions P;
  int N;
  if constexpr (DENSE) N = la.len.n[bi];
  else N = a.lens[bi];
  if (DENSE) {
    P.P = N; P.nx = N; P.sink = 0; P.Nc = 0; P.nK = 0; P.kp = nullptr;
    return P;
  }
  const int Nc = (N / a.C) * a.C;
  // tail [Nc, Ne): the partial chunk, and for a block of queries the block's rows up to
  // and including the unit's own
  const int Ne = a.qtail ? N + unit_query(u, a.hr, a.Hkv, a.Tq) + 1 : N;
  const int nK = a.kept_count[u];
  const int32_t* kp = a.kept + (int64_t)u * a.cap1;
  const int sink = (Nc > 0 && (nK == 0 || kp[0] != 0)) ? 1 : 0;
  P.sink = sink;
  P.nx = sink + (Ne - Nc);
  P.P = P.nx + nK * a.C;
  P.Nc = Nc;
  P.nK = nK;
  P.kp = kp;
  return P;
}

constexpr int ATT_STEP = 32;  // positions per wave step

// Token lookup for one wave's window of ATT_STEP positions starting at p0.  The chunk
// ids the window touches (at most ATT_STEP / C + 2) are fetched with one load, lane j
// holding the j-th, and handed to the lanes that need them with a shuffle, so a window's
// K/V addresses cost one dependent load that can be issued windows ahead.  PO2: the chunk
// is a power of two (Cshift >= 0) and every lookup is shifts and selects, with no branch
// between the K/V loads of a window (the generic form divides by C and returns early).
template <bool DENSE, bool PO2 = false>
struct Window {
  int ids;  // this lane's chunk id (lane j: chunk cb + j of the window)

  __device__ static __forceinline__ int first_chunk(const Positions& P, int p0, int C, int Cshift) {
    const int q = p0 - P.nx;
    if constexpr (PO2) return max(q, 0) >> Cshift;
    if (q <= 0) return 0;
    return Cshift >= 0 ? (q >> Cshift) : q / C;
  }
  // Issues the id load of window p0 (nothing to load in dense mode).
  __device__ __forceinline__ void fetch(const Positions& P, int p0, int end, int C, int Cshift, int lane) {
    if (DENSE) { ids = 0; return; }
    const int nwin = ATT_STEP / C + 2;
    const int k = first_chunk(P, p0, C, Cshift) + lane;
    ids = (lane < nwin && p0 < end && k < P.nK) ? P.kp[k] : 0;
  }
  // Token of position p of window p0; positions at or past `end` map to token 0 (read, masked).
  // Every lane of the wave must call this together (it shuffles).
  __device__ __forceinline__ int token(const Positions& P, int p0, int p, int end, int C, int Cshift) const {
    if (DENSE) return p < end ? p : 0;
    if constexpr (PO2) {
      const int q = p - P.nx;
      const int qc = max(q, 0);
      const int src = min(max((qc >> Cshift) - first_chunk(P, p0, C, Cshift), 0), 63);
      const int id = __shfl(ids, src);
      const int ctok = (id << Cshift) + (qc & ((1 << Cshift) - 1));
      const int xtok = (P.sink && p == 0) ? 0 : P.Nc + p - P.sink;  // sink, then the tail
      const int tok = q < 0 ? xtok : ctok;
      return p < end ? tok : 0;
    }
    const int q = p - P.nx;
    int k = 0;
    if (q > 0) k = Cshift >= 0 ? (q >> Cshift) : q / C;
    const int src = min(max(k - first_chunk(P, p0, C, Cshift), 0), 63);
    const int id = __shfl(ids, src);
    if (p >= end) return 0;
    if (q < 0) return (P.sink && p == 0) ? 0 : P.Nc + p - P.sink;
    return Cshift >= 0 ? (id << Cshift) + (q & ((1 << Cshift) - 1)) : id * C + (q - k * C);
  }
};

// ---------------------------------------------------------------- P.V, per storage type

template <typename T, int D> struct PV;

// bf16: V tile [32][D] staged in this wave's LDS region, read transposed.
template <int D> struct PV<__bf16, D> {
  static constexpr int LDS_STRIDE = D + 8;                    // elements; keeps 16-B rows, spreads banks
  static constexpr int LDS_ELEMS = ATT_STEP * LDS_STRIDE;     // per wave
  static constexpr int ND = D / 16;
  typedef bf16x8_t vfrag[ATT_STEP * D / 8 / 64];              // 16-B pieces per lane
  static constexpr int CPR = D / 8;                           // 16-B chunks per row
  static constexpr int RPI = 64 / CPR;                        // rows per load instruction
  static constexpr int NLD = ATT_STEP / RPI;

  template <class WIN>
  __device__ static __forceinline__ void load(vfrag& vf, const __bf16* Vb, const Positions& P, const WIN& win,
                                              int p0, int end, int C, int Cshift, int lane) {
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      const int ts = RPI * k + lane / CPR;
      const int tok = win.token(P, p0, p0 + ts, end, C, Cshift);
      vf[k] = __builtin_nontemporal_load((const bf16x8_t*)(Vb + (int64_t)tok * D + 8 * (lane % CPR)));
    }
  }
  __device__ static __forceinline__ void stage(const vfrag& vf, __bf16* lds, int lane) {
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      const int ts = RPI * k + lane / CPR;
      *(bf16x8_t*)(lds + ts * LDS_STRIDE + 8 * (lane % CPR)) = vf[k];
    }
  }
  // o[dt] += V^T(d-tile dt) * P^T, k-slot e of lane group grp <-> token e<4 ? 4grp+e : 16+4grp+e-4
  __device__ static __forceinline__ void mma(f32x4_t (&o)[ND], const __bf16* lds, const float (&p)[2][4], int lane) {
    const int row = lane & 15, grp = lane >> 4;
    // P = hi + lo, each half rounded to nearest even by the packed hardware conversion
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x8_t ph, pl;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const f32x2_t x = {p[e >> 2][e & 3], p[(e + 1) >> 2][(e + 1) & 3]};
      const bf16x2_t h = __builtin_convertvector(x, bf16x2_t);
      const bf16x2_t l = __builtin_convertvector(x - __builtin_convertvector(h, f32x2_t), bf16x2_t);
      ph[e] = h[0];
      ph[e + 1] = h[1];
      pl[e] = l[0];
      pl[e + 1] = l[1];
    }
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      bf16x8_t va;
      const __bf16* col = lds + dt * 16 + row;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int ts = (e < 4) ? 4 * grp + e : 16 + 4 * grp + (e - 4);
        va[e] = col[ts * LDS_STRIDE];
      }
      o[dt] = Mf<__bf16>::mma(va, ph, o[dt]);
      o[dt] = Mf<__bf16>::mma(va, pl, o[dt]);
    }
  }
};

// f32: one element per lane per k-step, V read straight from memory.
template <int D> struct PV<float, D> {
  static constexpr int LDS_ELEMS = 0;
  static constexpr int ND = D / 16;
  typedef float vfrag[2][4][ND];
  template <class WIN>
  __device__ static __forceinline__ void load(vfrag& vf, const float* Vb, const Positions& P, const WIN& win,
                                              int p0, int end, int C, int Cshift, int lane) {
    const int row = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int p = p0 + 16 * t + 4 * grp + jj;
        const int tok = win.token(P, p0, p, end, C, Cshift);
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) vf[t][jj][dt] = Vb[(int64_t)tok * D + dt * 16 + row];
      }
  }
  __device__ static __forceinline__ void stage(const vfrag&, float*, int) {}
  __device__ static __forceinline__ void mma(f32x4_t (&o)[ND], const vfrag& vf, const float (&p)[2][4]) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) o[dt] = Mf<float>::mma(vf[t][jj][dt], p[t][jj], o[dt]);
  }
};

// Two waves per SIMD for bf16 K/V (at most 256 registers per lane; a second workgroup per
// compute unit keeps twice the K/V loads in flight).
template <typename T, int D, bool DENSE, bool UNI, bool PO2 = false>
__global__ __launch_bounds__(256, sizeof(T) == 2 ? 2 : 1) void zha_attend_kernel(AttArgs a, LensArg<DENSE> la) {
  typedef Mf<T> M;
  typedef PV<T, D> PVT;
  constexpr bool TD = DENSE;  // positions are tokens
  typedef Window<TD, PO2 && !DENSE> Win;
  constexpr int NK = D / M::KPER;
  constexpr int ND = D / 16;
  constexpr int LDS_WAVE = PVT::LDS_ELEMS > 0 ? PVT::LDS_ELEMS : 1;
  constexpr int COMB_BYTES = 4 * 16 * D * 4 + 2 * 4 * 16 * 4;
  constexpr int STAGE_BYTES = 4 * LDS_WAVE * (int)sizeof(T);
  constexpr int SMEM = COMB_BYTES > STAGE_BYTES ? COMB_BYTES : STAGE_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane & 15, grp = lane >> 4;
  // u: routing unit, of G query heads; up: its (sequence, KV head) unit.  Units are numbered
  // (sequence, query, KV head, head group), so the unit's first query head is u * G.
  // UNI: lane column `col` is head jcol of unit u; the group reads token 0, the tail up to
  // its last query and the chunks some unit of the group kept, and a column takes token 0,
  // the tokens of its unit's kept chunks and its own tail [Nc, Ne).
  const int G = a.G;
  const int col = row;
  int u, up, bi, jcol, Ne = 0, Nc = 0;
  bool colok;
  Positions P;
  if constexpr (UNI) {
    up = blockIdx.y / a.NTC;
    const int tc = blockIdx.y - up * a.NTC, g = up % a.Hkv;
    bi = up / a.Hkv;
    const int per_t = a.hr * G;
    const int tt = col / per_t, h = (col / G) % a.hr, tq = tc * a.TS + tt;
    colok = tt < a.TS && tq < a.Tq;
    u = ((bi * a.Tq + min(tq, a.Tq - 1)) * a.Hkv + g) * a.hr + h;
    jcol = col % G;
    const int N = a.lens[bi];
    Nc = (N / a.C) * a.C;
    Ne = a.qtail ? N + min(tq, a.Tq - 1) + 1 : N;
    const int tlast = min(tc * a.TS + a.TS, a.Tq) - 1;  // the group's last query
    const int Nend = a.qtail ? N + tlast + 1 : N;
    const int nK = a.ucount[blockIdx.y];
    const int32_t* kp = a.ulist + (int64_t)blockIdx.y * a.cap1;
    P.sink = (Nc > 0 && (nK == 0 || kp[0] != 0)) ? 1 : 0;
    P.nx = P.sink + (Nend - Nc);
    P.P = P.nx + nK * a.C;
    P.Nc = Nc;
    P.nK = nK;
    P.kp = kp;
  } else {
    u = blockIdx.y;
    up = plane_unit(u, a.hr, a.Hkv, a.Tq);
    bi = up / a.Hkv;
    colok = row < G;
    jcol = row;
    P = unit_positions<DENSE>(a, la, u, bi);
  }
  const u64* kr1 = UNI ? a.krank + (int64_t)u * a.cap1 : nullptr;
  const uint32_t stamp = UNI ? a.route_ctr[0] : 0u;
  // Blocks of 4 * ATT_STEP positions are dealt to the workgroups in turn, so the unit's
  // workgroups read neighbouring K/V rows at any moment.
  constexpr int WSTEP = 4 * ATT_STEP;
  const int start = blockIdx.x * WSTEP;
  const int gstep = a.W * WSTEP;
  const int end = P.P;

  const int64_t kvoff = (int64_t)up * a.T * D;
  const T* Kb = (const T*)a.K + kvoff;
  const T* Vb = (const T*)a.V + kvoff;

  typename M::frag qf[NK];
  {
    const T* qp = (const T*)a.q + ((int64_t)u * G + jcol) * D + grp * M::EPL;
#pragma unroll
    for (int s = 0; s < NK; ++s) qf[s] = colok ? M::load(qp + s * M::KPER) : M::zero();
  }
  T* lds = (T*)smem + wave * LDS_WAVE;

  f32x4_t o[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) o[dt] = (f32x4_t){0.0f, 0.0f, 0.0f, 0.0f};
  float mrun = -INFINITY, lrun = 0.0f;

  // One window: K rows of the two 16-token tiles (lane row r -> position p0 + 16t + r) and
  // the V tile, loaded into registers.
  auto load_kv = [&](typename M::frag (&kf)[2][NK], typename PVT::vfrag& vf, const Win& win, int p0) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int tok = win.token(P, p0, p0 + 16 * t + row, end, a.C, a.Cshift);
      const T* kr = Kb + (int64_t)tok * D + grp * M::EPL;
#pragma unroll
      for (int s = 0; s < NK; ++s) kf[t][s] = M::load_stream(kr + s * M::KPER);
    }
    PVT::load(vf, Vb, P, win, p0, end, a.C, a.Cshift, lane);
  };
  // UNI: stamps (the high words of the kept-rank entries) of the chunks of this lane's
  // positions p0 + 16t + 4grp + jj for the lane's column unit (0 outside the chunk part).
  // Every lane calls this together (the token lookup shuffles).
  // A lane's four consecutive positions lie in at most three consecutive kept chunks (two when
  // C >= 3): three stamps per group of four, from the window's chunk ids (a stamp needs no
  // token), loaded unconditionally (ids outside the list are 0, a readable entry).
  auto fetch_rank = [&](const Win& win, int p0, uint32_t (&rk)[2][4]) {
    const int cb = Win::first_chunk(P, p0, a.C, a.Cshift);
    auto lidx = [&](int q) { return q > 0 ? (a.Cshift >= 0 ? (q >> a.Cshift) : q / a.C) : 0; };
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int pg = p0 + 16 * t + 4 * grp;
      const int k0 = lidx(pg - P.nx), k3 = lidx(pg + 3 - P.nx), k1 = min(k0 + 1, k3);
      uint32_t st[3];
      const int kc[3] = {k0, k1, k3};
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const int id = __shfl(win.ids, min(max(kc[i] - cb, 0), 63));
        st[i] = ((const uint32_t*)(kr1 + id))[1];
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int p = pg + jj;
        const bool need = colok && p < end && p >= P.nx;
        const int kj = lidx(p - P.nx);
        const uint32_t sj = kj == k0 ? st[0] : (kj == k1 ? st[1] : st[2]);
        rk[t][jj] = need ? sj : 0u;
      }
    }
  };
  // UNI: bit 4t + jj: position p0 + 16t + 4grp + jj is in the column's set: token 0 always,
  // the tail up to the column's own end, a chunk token when the column's unit kept it
  const bool chunk0 = UNI && Nc > 0 && !P.sink;  // token 0 is the union list's first chunk token
  auto member_bits = [&](int p0, const uint32_t (&rk)[2][4]) {
    uint32_t bits = 0;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int p = p0 + 16 * t + 4 * grp + jj;
        bool in;
        if (p < P.nx) {
          const int tok = (P.sink && p == 0) ? 0 : P.Nc + p - P.sink;
          in = tok == 0 || tok < Ne;
        } else {
          in = p < end && (rk[t][jj] == stamp || (p == P.nx && chunk0));
        }
        bits |= (colok && in) ? (1u << (4 * t + jj)) : 0u;
      }
    return bits;
  };
  // Online-softmax update with one loaded window.
  auto compute = [&](const typename M::frag (&kf)[2][NK], const typename PVT::vfrag& vf, int p0, uint32_t bits) {
    // S^T = K Q^T: lane holds tokens 16t + 4grp + jj for head `row`
    float z[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < NK; ++s) acc = M::mma(kf[t][s], qf[s], acc);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int p = p0 + 16 * t + 4 * grp + jj;
        const bool in = UNI ? ((bits >> (4 * t + jj)) & 1u) != 0 : p < end;
        z[t][jj] = in ? acc[jj] * a.scale_log2 : -INFINITY;
      }
    }
    float mloc = fmaxf(fmaxf(fmaxf(z[0][0], z[0][1]), fmaxf(z[0][2], z[0][3])),
                       fmaxf(fmaxf(z[1][0], z[1][1]), fmaxf(z[1][2], z[1][3])));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float mnew = fmaxf(mrun, mloc);
    // branch-free: a column with nothing in its set so far (mnew = -inf) takes 0 as its
    // maximum, so alpha and every p are exp2(-inf) = 0 (its o and l are still 0)
    const float msafe = mnew == -INFINITY ? 0.0f : mnew;
    const float alpha = zexp2(mrun - msafe);
    float pr[2][4];
    float psum = 0.0f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        pr[t][jj] = zexp2(z[t][jj] - msafe);
        psum += pr[t][jj];
      }
    lrun = lrun * alpha + psum;
    mrun = mnew;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) o[dt] *= alpha;
    if constexpr (PVT::LDS_ELEMS > 0) {
      PVT::stage(vf, lds, lane);
      PVT::mma(o, lds, pr, lane);
    } else {
      PVT::mma(o, vf, pr);
    }
  };

  // Software pipeline over the wave's windows p0, p0 + gstep, ...: while window i is
  // computed, the K/V loads of window i+1 and the chunk ids of window i+2 are in flight.
  // The two register buffers alternate by unrolling the loop twice.
  int p0 = start + wave * ATT_STEP;
  Win w0, w1;
  typename M::frag kA[2][NK], kB[2][NK];
  typename PVT::vfrag vA, vB;
  if constexpr (UNI) {
    // the sparse pipeline over the union's positions, with the column stamps of each window
    // fetched one window ahead (they depend on the window's chunk ids)
    uint32_t rA[2][4], rB[2][4];
    w0.fetch(P, p0, end, a.C, a.Cshift, lane);
    w1.fetch(P, p0 + gstep, end, a.C, a.Cshift, lane);
    fetch_rank(w0, p0, rA);
    if (p0 < end) load_kv(kA, vA, w0, p0);
    while (p0 < end) {
      fetch_rank(w1, p0 + gstep, rB);
      w0.fetch(P, p0 + 2 * gstep, end, a.C, a.Cshift, lane);
      load_kv(kB, vB, w1, p0 + gstep);
      compute(kA, vA, p0, member_bits(p0, rA));
      p0 += gstep;
      if (p0 >= end) break;
      fetch_rank(w0, p0 + gstep, rA);
      w1.fetch(P, p0 + 2 * gstep, end, a.C, a.Cshift, lane);
      load_kv(kA, vA, w0, p0 + gstep);
      compute(kB, vB, p0, member_bits(p0, rB));
      p0 += gstep;
    }
  } else {
    w0.fetch(P, p0, end, a.C, a.Cshift, lane);
    w1.fetch(P, p0 + gstep, end, a.C, a.Cshift, lane);
    if (p0 < end) load_kv(kA, vA, w0, p0);
    while (p0 < end) {
      w0.fetch(P, p0 + 2 * gstep, end, a.C, a.Cshift, lane);
      load_kv(kB, vB, w1, p0 + gstep);
      compute(kA, vA, p0, 0u);
      p0 += gstep;
      if (p0 >= end) break;
      w1.fetch(P, p0 + 2 * gstep, end, a.C, a.Cshift, lane);
      load_kv(kA, vA, w0, p0 + gstep);
      compute(kB, vB, p0, 0u);
      p0 += gstep;
    }
  }
  // per-head sum over the four lane groups, then combine the four waves through LDS
  lrun += __shfl_xor(lrun, 16);
  lrun += __shfl_xor(lrun, 32);
  __syncthreads();  // the staging area is reused below
  float* so = (float*)smem;                    // [4][16][D]
  float* sm = so + 4 * 16 * D;                 // [4][16]
  float* sl = sm + 4 * 16;                     // [4][16]
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) so[(wave * 16 + row) * D + dt * 16 + 4 * grp + jj] = o[dt][jj];
  if (grp == 0) { sm[wave * 16 + row] = mrun; sl[wave * 16 + row] = lrun; }
  __shared__ int s_rec[16];  // each column's (unit, workgroup, head) record; -1: no query head
  if (wave == 0 && grp == 0) s_rec[col] = colok ? (u * a.W + (int)blockIdx.x) * G + jcol : -1;
  __syncthreads();
  float* pml0 = a.part + (int64_t)a.U * a.W * G * D;
  const int ncol = UNI ? 16 : G;
  for (int i = threadIdx.x; i < ncol * D; i += 256) {
    const int h = i / D, dd = i % D;
    const int rec = s_rec[h];
    if (rec < 0) continue;
    float* po = a.part + (int64_t)rec * D;
    float* pml = pml0 + (int64_t)rec * 2;
    float Mx = -INFINITY;
    for (int w = 0; w < 4; ++w) Mx = fmaxf(Mx, sm[w * 16 + h]);
    float acc = 0.0f, l = 0.0f;
    if (Mx != -INFINITY) {
      for (int w = 0; w < 4; ++w) {
        const float f = zexp2(sm[w * 16 + h] - Mx);
        acc += f * so[(w * 16 + h) * D + dd];
        l += f * sl[w * 16 + h];
      }
    }
    po[dd] = acc;
    if (dd == 0) {
      pml[0] = Mx;
      pml[1] = l;
    }
  }
}

// Union attention over 16 * CT query heads of one group (bf16): every stage of 128 / CT
// positions is loaded once by the whole workgroup into LDS (two buffers; the next two
// stages' loads in flight in registers while one is computed), and wave w multiplies its
// window (slot w / CT) with its 16 columns (tile w % CT), each column's softmax masked to
// its own unit's set as in zha_attend_kernel<..., UNI>.
template <int D, int CT, bool PO2 = false>
__global__ __launch_bounds__(256, 2) void zha_attend_union_lds_kernel(AttArgs a) {
  typedef Mf<__bf16> M;
  typedef PV<__bf16, D> PVT;
  constexpr int NK = D / M::KPER, ND = D / 16;
  constexpr int NWS = 4 / CT;                 // windows of ATT_STEP positions per stage
  constexpr int TOK = ATT_STEP * NWS;         // positions per stage
  constexpr int KST = PVT::LDS_STRIDE;        // LDS row stride (elements), K and V alike
  constexpr int CPR = D / 8;                  // 16-byte pieces per row
  constexpr int NLD = TOK * CPR / 256;        // pieces per thread per matrix and stage
  constexpr int BUF = TOK * KST;              // elements of one matrix in one buffer
  constexpr int COMB = 4 * 16 * D * 4 + 2 * 4 * 16 * 4;
  constexpr int SMEM = 4 * BUF * 2 > COMB ? 4 * BUF * 2 : COMB;
  static_assert(NLD * 256 == TOK * CPR, "whole pieces per thread");
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  __bf16* skv = (__bf16*)smem;                // buffer b: K at 2b * BUF, V at (2b + 1) * BUF

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = lane & 15, grp = lane >> 4;
  const int ct = wave % CT, ws = wave / CT;
  const int G = a.G;
  const int col = 16 * ct + row;
  // the lane's column: head jcol of routing unit u (query tq of the block)
  const int up = blockIdx.y / a.NTC;
  const int tc = blockIdx.y - up * a.NTC, g = up % a.Hkv, bi = up / a.Hkv;
  const int per_t = a.hr * G;
  const int tt = col / per_t, h = (col / G) % a.hr, tq = tc * a.TS + tt;
  const bool colok = tt < a.TS && tq < a.Tq;
  const int u = ((bi * a.Tq + min(tq, a.Tq - 1)) * a.Hkv + g) * a.hr + h;
  const int jcol = col % G;
  const int N = a.lens[bi];
  const int Nc = (N / a.C) * a.C;
  const int Ne = a.qtail ? N + min(tq, a.Tq - 1) + 1 : N;
  const int tlast = min(tc * a.TS + a.TS, a.Tq) - 1;
  const int Nend = a.qtail ? N + tlast + 1 : N;
  Positions P;
  P.nK = a.ucount[blockIdx.y];
  P.kp = a.ulist + (int64_t)blockIdx.y * a.cap1;
  P.sink = (Nc > 0 && (P.nK == 0 || P.kp[0] != 0)) ? 1 : 0;
  P.nx = P.sink + (Nend - Nc);
  P.P = P.nx + P.nK * a.C;
  P.Nc = Nc;
  const int end = P.P;
  const bool chunk0 = Nc > 0 && !P.sink;  // token 0 is the list's first chunk token
  const u64* kr1 = a.krank + (int64_t)u * a.cap1;
  const uint32_t stamp = a.route_ctr[0];
  const int64_t kvoff = (int64_t)up * a.T * D;
  const __bf16* Kb = (const __bf16*)a.K + kvoff;
  const __bf16* Vb = (const __bf16*)a.V + kvoff;

  typename M::frag qf[NK];
  {
    const __bf16* qp = (const __bf16*)a.q + ((int64_t)u * G + jcol) * D + grp * M::EPL;
#pragma unroll
    for (int s = 0; s < NK; ++s) qf[s] = colok ? M::load(qp + s * M::KPER) : M::zero();
  }
  f32x4_t o[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) o[dt] = (f32x4_t){0.0f, 0.0f, 0.0f, 0.0f};
  float mrun = -INFINITY, lrun = 0.0f;

  const int start = blockIdx.x * TOK;
  const int gstep = a.W * TOK;
  // Chunk ids of the stage at ps: lane j holds the j-th kept chunk its positions touch, read
  // from a clamped index, so the stage's tokens cost one load that no branch guards (a
  // guarded load makes the compiler wait for every load in flight).  The clamped entry lies
  // inside the group's list row whatever the count; a group with an empty list (a sequence
  // without a complete chunk) has no written entry there, so its ids are taken as chunk 0,
  // whose rank entry is always readable (only positions of the chunk part use them).
  static_assert(TOK / 2 + 2 <= 64, "a stage touches at most 64 chunks (C >= 2)");
  const int nidx = max(P.nK - 1, 0);
  const bool csh = PO2 || a.Cshift >= 0;  // PO2: the chunk is a power of two (no division)
  auto first_chunk = [&](int ps) {
    const int q = ps - P.nx;
    return q <= 0 ? 0 : (csh ? (q >> a.Cshift) : q / a.C);
  };
  auto stage_ids = [&](int ps) -> int {
    const int x = P.kp[min(first_chunk(ps) + lane, nidx)];
    return P.nK > 0 ? x : 0;
  };
  // token of position p of the stage at ps (positions at or past the end: token 0); every
  // lane calls this together (it shuffles)
  auto stage_token = [&](int ids, int ps, int p) -> int {
    const int q = p - P.nx;
    const int k = q > 0 ? (csh ? (q >> a.Cshift) : q / a.C) : 0;
    const int id = __shfl(ids, min(max(k - first_chunk(ps), 0), 63));
    const int ct = csh ? (id << a.Cshift) + (q & ((1 << a.Cshift) - 1)) : id * a.C + (q - k * a.C);
    const int pre = (P.sink && p == 0) ? 0 : P.Nc + p - P.sink;
    return p >= end ? 0 : (q < 0 ? pre : ct);
  };
  // tokens of this thread's rows of the stage at ps
  auto tokens = [&](int ps, int ids, int (&tk)[NLD]) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) tk[i] = stage_token(ids, ps, ps + (tid + 256 * i) / CPR);
  };
  auto issue = [&](const int (&tk)[NLD], bf16x8_t (&kr)[NLD], bf16x8_t (&vr)[NLD]) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int pc = (tid + 256 * i) % CPR;
      kr[i] = M::load_stream(Kb + (int64_t)tk[i] * D + 8 * pc);
      vr[i] = M::load_stream(Vb + (int64_t)tk[i] * D + 8 * pc);
    }
  };
  auto store = [&](int b, const bf16x8_t (&kr)[NLD], const bf16x8_t (&vr)[NLD]) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int c = tid + 256 * i, r = c / CPR, pc = c % CPR;
      *(bf16x8_t*)(skv + (2 * b) * BUF + r * KST + 8 * pc) = kr[i];
      *(bf16x8_t*)(skv + (2 * b + 1) * BUF + r * KST + 8 * pc) = vr[i];
    }
  };
  // stamps of the chunks of this lane's positions in its window of the stage at ps, for the
  // lane's column unit (0 outside the chunk part).  A lane's four consecutive positions lie in
  // at most three consecutive kept chunks (two when C >= 3), so three stamps are loaded per
  // group of four, straight from the chunk ids (a stamp needs no token); the loads are
  // unconditional (every id is a listed chunk, or chunk 0 for an empty list: readable).
  auto fetch_rank = [&](int ps, int ids, uint32_t (&rk)[2][4]) {
    const int cb = first_chunk(ps);
    auto lidx = [&](int q) { return q > 0 ? (csh ? (q >> a.Cshift) : q / a.C) : 0; };
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int p0 = ps + ws * ATT_STEP + 16 * t + 4 * grp;
      const int k0 = lidx(p0 - P.nx), k3 = lidx(p0 + 3 - P.nx), k1 = min(k0 + 1, k3);
      uint32_t st[3];
      const int kc[3] = {k0, k1, k3};
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const int id = __shfl(ids, min(max(kc[i] - cb, 0), 63));
        st[i] = ((const uint32_t*)(kr1 + id))[1];
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int p = p0 + jj;
        const bool need = colok && p < end && p >= P.nx;
        const int kj = lidx(p - P.nx);
        const uint32_t sj = kj == k0 ? st[0] : (kj == k1 ? st[1] : st[2]);
        rk[t][jj] = need ? sj : 0u;
      }
    }
  };
  auto member_bits = [&](int ps, const uint32_t (&rk)[2][4]) {
    uint32_t bits = 0;
    const int w0 = ps + ws * ATT_STEP;
    if (w0 > P.nx && w0 + ATT_STEP <= end) {
      // the whole window lies in the chunk part, past its first position: the stamp decides
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) bits |= (colok && rk[t][jj] == stamp) ? (1u << (4 * t + jj)) : 0u;
      return bits;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int p = ps + ws * ATT_STEP + 16 * t + 4 * grp + jj;
        bool in;
        if (p < P.nx) {
          const int tok = (P.sink && p == 0) ? 0 : P.Nc + p - P.sink;
          in = tok == 0 || tok < Ne;
        } else {
          in = p < end && (rk[t][jj] == stamp || (p == P.nx && chunk0));
        }
        bits |= (colok && in) ? (1u << (4 * t + jj)) : 0u;
      }
    return bits;
  };
  // online-softmax update of this wave's columns with its window of buffer b
  auto compute = [&](int b, uint32_t bits) {
    const __bf16* sk = skv + (2 * b) * BUF + ws * ATT_STEP * KST;
    const __bf16* sv = skv + (2 * b + 1) * BUF + ws * ATT_STEP * KST;
    float z[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < NK; ++s)
        acc = M::mma(*(const bf16x8_t*)(sk + (16 * t + row) * KST + s * M::KPER + grp * M::EPL), qf[s], acc);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        z[t][jj] = ((bits >> (4 * t + jj)) & 1u) ? acc[jj] * a.scale_log2 : -INFINITY;
    }
    float mloc = fmaxf(fmaxf(fmaxf(z[0][0], z[0][1]), fmaxf(z[0][2], z[0][3])),
                       fmaxf(fmaxf(z[1][0], z[1][1]), fmaxf(z[1][2], z[1][3])));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float mnew = fmaxf(mrun, mloc);
    // branch-free: a column with nothing in its set so far (mnew = -inf) takes 0 as its
    // maximum, so alpha and every p are exp2(-inf) = 0 (its o and l are still 0)
    const float msafe = mnew == -INFINITY ? 0.0f : mnew;
    const float alpha = zexp2(mrun - msafe);
    float pr[2][4];
    float psum = 0.0f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        pr[t][jj] = zexp2(z[t][jj] - msafe);
        psum += pr[t][jj];
      }
    lrun = lrun * alpha + psum;
    mrun = mnew;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) o[dt] *= alpha;
    PVT::mma(o, sv, pr, lane);
  };

  // pipeline over the stages ps, ps + gstep, ...: while the stage at ps (in LDS buffer b) is
  // computed, the K/V of the next two stages are loading into registers (stored to LDS one
  // stage ahead of use), the column stamps of the next stage and the chunk ids of the stage
  // after those are in flight.  Every lookup is issued before the K/V loads of its iteration
  // and consumed in a later one, so waiting for a lookup never drains the K/V loads.
  // Register sets rotate with the stage index mod 3.
  bf16x8_t kk[3][NLD], vv[3][NLD];
  int ids[3];
  uint32_t rk[3][2][4];
  int ps = start, b = 0;
  ids[0] = stage_ids(ps);
  ids[1] = stage_ids(ps + gstep);
  ids[2] = stage_ids(ps + 2 * gstep);
  {
    int tk[NLD];
    tokens(ps, ids[0], tk);
    issue(tk, kk[0], vv[0]);
    tokens(ps + gstep, ids[1], tk);
    issue(tk, kk[1], vv[1]);
  }
  fetch_rank(ps, ids[0], rk[0]);
  store(0, kk[0], vv[0]);
  __syncthreads();
  auto iter = [&](auto J) {
    constexpr int j = decltype(J)::value, j1 = (j + 1) % 3, j2 = (j + 2) % 3;  // stages ps, +1, +2
    ids[j] = stage_ids(ps + 3 * gstep);
    fetch_rank(ps + gstep, ids[j1], rk[j1]);
    {
      int tk[NLD];
      tokens(ps + 2 * gstep, ids[j2], tk);
      issue(tk, kk[j2], vv[j2]);
    }
    compute(b, member_bits(ps, rk[j]));
    store(b ^ 1, kk[j1], vv[j1]);      // stage ps + gstep
    __syncthreads();
    b ^= 1;
    ps += gstep;
  };
  while (ps < end) {
    iter(std::integral_constant<int, 0>{});
    if (ps >= end) break;
    iter(std::integral_constant<int, 1>{});
    if (ps >= end) break;
    iter(std::integral_constant<int, 2>{});
  }
  // per-column partials: lane groups, then the waves of the column's tile
  lrun += __shfl_xor(lrun, 16);
  lrun += __shfl_xor(lrun, 32);
  float* so = (float*)smem;                    // [4][16][D]
  float* sm = so + 4 * 16 * D;                 // [4][16]
  float* sl = sm + 4 * 16;                     // [4][16]
  __shared__ int s_rec[16 * CT];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) so[(wave * 16 + row) * D + dt * 16 + 4 * grp + jj] = o[dt][jj];
  if (grp == 0) { sm[wave * 16 + row] = mrun; sl[wave * 16 + row] = lrun; }
  if (ws == 0 && grp == 0) s_rec[col] = colok ? (u * a.W + (int)blockIdx.x) * G + jcol : -1;
  __syncthreads();
  float* pml0 = a.part + (int64_t)a.U * a.W * G * D;
  for (int i = tid; i < 16 * CT * D; i += 256) {
    const int c = i / D, dd = i % D, c0 = c >> 4, hh = c & 15;
    const int rec = s_rec[c];
    if (rec < 0) continue;
    float Mx = -INFINITY;
    for (int w = c0; w < 4; w += CT) Mx = fmaxf(Mx, sm[w * 16 + hh]);
    float acc = 0.0f, l = 0.0f;
    if (Mx != -INFINITY) {
      for (int w = c0; w < 4; w += CT) {
        const float f = zexp2(sm[w * 16 + hh] - Mx);
        acc += f * so[(w * 16 + hh) * D + dd];
        l += f * sl[w * 16 + hh];
      }
    }
    a.part[(int64_t)rec * D + dd] = acc;
    if (dd == 0) {
      pml0[(int64_t)rec * 2] = Mx;
      pml0[(int64_t)rec * 2 + 1] = l;
    }
  }
}

// Merges the W partials of each (unit, head): the maximum first, then the scaled sums,
// each thread summing a fixed subset of workgroups and the subsets combined in order.
constexpr int MERGE_THREADS = 1024;
constexpr int MERGE_BATCH = 4;

template <int D>
__global__ __launch_bounds__(MERGE_THREADS) void zha_merge_kernel(const float* part, int U, int W, int G, float* out,
                                                                  float* lse) {
  constexpr int TPR = D / 4;                  // threads per record (4 floats each)
  constexpr int NGRP = MERGE_THREADS / TPR;   // workgroup subsets
  const int h = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const float* po = part + ((int64_t)u * W * G + h) * D;                            // record w at po + w*G*D
  const float* pml = part + (int64_t)U * W * G * D + ((int64_t)u * W * G + h) * 2;  // at pml + w*G*2
  __shared__ float s_red[MERGE_THREADS / 64];
  __shared__ float4 s_o[NGRP][TPR];
  __shared__ float s_l[NGRP];
  const int j = tid / TPR, c = tid % TPR;
  // thread (j, c) takes records j, j + NGRP, ... in batches; the first batch is in flight
  // while the maximum is formed
  float2 ml[MERGE_BATCH];
  float4 v[MERGE_BATCH];
  auto load_batch = [&](int w0) {
#pragma unroll
    for (int k = 0; k < MERGE_BATCH; ++k) {  // unconditional loads from clamped records (W >= 1)
      const int w = w0 + k * NGRP, wc = min(w, W - 1);
      const float2 x = *(const float2*)(pml + (int64_t)wc * G * 2);
      v[k] = *(const float4*)(po + (int64_t)wc * G * D + 4 * c);
      ml[k] = w < W ? x : make_float2(0.0f, 0.0f);  // y = 0: the record is skipped
    }
  };
  load_batch(j);
  float mx = -INFINITY;
  for (int w = tid; w < W; w += MERGE_THREADS) {
    const float2 r = *(const float2*)(pml + (int64_t)w * G * 2);
    if (r.y > 0.0f) mx = fmaxf(mx, r.x);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if (lane == 0) s_red[wave] = mx;
  __syncthreads();
  float M = s_red[0];
  for (int k = 1; k < MERGE_THREADS / 64; ++k) M = fmaxf(M, s_red[k]);
  float4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  float lsum = 0.0f;
  for (int w0 = j; w0 < W; w0 += NGRP * MERGE_BATCH) {
    if (w0 > j) load_batch(w0);
#pragma unroll
    for (int k = 0; k < MERGE_BATCH; ++k) {
      if (ml[k].y > 0.0f) {
        const float f = zexp2(ml[k].x - M);
        acc.x += f * v[k].x; acc.y += f * v[k].y; acc.z += f * v[k].z; acc.w += f * v[k].w;
        lsum += f * ml[k].y;
      }
    }
  }
  s_o[j][c] = acc;
  if (c == 0) s_l[j] = lsum;
  __syncthreads();
  if (tid < TPR) {
    float4 o = s_o[0][tid];
    float L = s_l[0];
    for (int k = 1; k < NGRP; ++k) {
      const float4 v = s_o[k][tid];
      o.x += v.x; o.y += v.y; o.z += v.z; o.w += v.w;
      L += s_l[k];
    }
    const int64_t oh = (int64_t)u * G + h;  // units are numbered (sequence, KV head, head group)
    const float inv = 1.0f / L;
    *(float4*)(out + oh * D + 4 * tid) = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
    if (tid == 0) lse[oh] = (M + zlog2(L)) * ZHA_LN2;
  }
}

// rows: routing units, or groups of them (UNI)
template <typename T, int D, bool DENSE, bool UNI = false>
hipError_t launch_att(const AttArgs& a, const LensArg<DENSE>& la, int rows, hipStream_t s) {
  if constexpr (!DENSE) {
    if (a.Cshift >= 0) {
      hipLaunchKernelGGL((zha_attend_kernel<T, D, false, UNI, true>), dim3(a.W, rows), dim3(256), 0, s, a, la);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((zha_attend_kernel<T, D, DENSE, UNI>), dim3(a.W, rows), dim3(256), 0, s, a, la);
  return hipGetLastError();
}

template <int D>
hipError_t launch_merge(const AttArgs& a, int U, float* out, float* lse, hipStream_t s) {
  hipLaunchKernelGGL((zha_merge_kernel<D>), dim3(a.G, U), dim3(MERGE_THREADS), 0, s, (const float*)a.part, U, a.W,
                     a.G, out, lse);
  return hipGetLastError();
}

template <bool DENSE, bool UNI = false>
hipError_t launch_att_dt(const AttArgs& a, const LensArg<DENSE>& la, zha_dtype dt, int d, int rows, hipStream_t s) {
  if (dt == ZHA_BF16)
    return d == 64 ? launch_att<__bf16, 64, DENSE, UNI>(a, la, rows, s)
                   : launch_att<__bf16, 128, DENSE, UNI>(a, la, rows, s);
  return d == 64 ? launch_att<float, 64, DENSE, UNI>(a, la, rows, s)
                 : launch_att<float, 128, DENSE, UNI>(a, la, rows, s);
}

int cshift_of(int C) {
  if (C <= 0 || (C & (C - 1)) != 0) return -1;
  int s = 0;
  while ((1 << s) < C) ++s;
  return s;
}

}  // namespace

int zha_sparse_wgs(int U) {
  int w = 512 / (U > 0 ? U : 1);
  return w < 1 ? 1 : w;
}

int zha_dense_wgs(int U) {
  // one long-running workgroup per compute unit at small batch (measured best for the
  // in-order sweep of a unit's rows); at least 16 per unit at large batch
  int w = 256 / (U > 0 ? U : 1);
  return w < 16 ? 16 : w;
}

hipError_t zha_launch_attend(zha_tree* t, const void* q, const void* K, const void* V, float scale, float* out,
                             float* lse, hipStream_t s) {
  AttArgs a;
  a.q = q; a.K = K; a.V = V;
  a.kept = t->kept[1];
  a.kept_count = t->counts + (int64_t)(t->L + 2) * t->RU + t->RU;  // kept counts of level 1
  a.cap1 = t->cap[1];
  a.part = t->apart;
  a.W = t->WA;
  a.U = t->RU;
  a.hr = t->hr;
  a.Tq = t->Tq;
  a.qtail = t->multi ? 1 : 0;
  a.Hkv = t->desc.n_kv_heads;
  a.Hq = t->desc.n_q_heads;
  a.G = t->G / t->hr;
  a.C = t->C;
  a.Cshift = cshift_of(t->C);
  a.T = t->T;
  a.scale_log2 = scale * ZHA_LOG2E;
  a.lens = t->geo;
  // union attention: the groups of the route's union scoring, when it had one
  const int TS = zha_union_queries(t->R, t->G, t->Tq, t->hr, t->desc.dtype == ZHA_BF16);
  const bool uni = t->uni_route;
  const int CT = (TS * t->G + 15) / 16;  // column tiles of a union group
  a.krank = uni ? t->krank[1] : nullptr;
  a.route_ctr = t->route_ctr;
  a.ulist = t->ulist;
  a.ucount = t->ucount;
  a.TS = TS;
  a.NTC = uni ? (t->Tq + TS - 1) / TS : 1;
  const int rows = uni ? t->U * a.NTC : t->RU;
  if (uni) a.W = zha_sparse_wgs(rows);
  zha_time_begin(t, s, ZHA_K_ATTEND, 0);
  hipError_t e;
  if (uni && CT > 1) {  // bf16 (wider groups are formed for bf16 only): windows staged in LDS
    const bool p2 = a.Cshift >= 0;
    if (CT == 2)
      hipLaunchKernelGGL((t->d == 64 ? (p2 ? zha_attend_union_lds_kernel<64, 2, true> : zha_attend_union_lds_kernel<64, 2>)
                                     : (p2 ? zha_attend_union_lds_kernel<128, 2, true> : zha_attend_union_lds_kernel<128, 2>)),
                         dim3(a.W, rows), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((t->d == 64 ? (p2 ? zha_attend_union_lds_kernel<64, 4, true> : zha_attend_union_lds_kernel<64, 4>)
                                     : (p2 ? zha_attend_union_lds_kernel<128, 4, true> : zha_attend_union_lds_kernel<128, 4>)),
                         dim3(a.W, rows), dim3(256), 0, s, a);
    e = hipGetLastError();
  } else {
    e = uni ? launch_att_dt<false, true>(a, LensArg<false>{}, t->desc.dtype, t->d, rows, s)
            : launch_att_dt<false>(a, LensArg<false>{}, t->desc.dtype, t->d, rows, s);
  }
  if (e != hipSuccess) return e;
  zha_time_end(t, s, ZHA_K_ATTEND, 0);
  zha_time_begin(t, s, ZHA_K_MERGE, 0);
  e = t->d == 64 ? launch_merge<64>(a, t->RU, out, lse, s) : launch_merge<128>(a, t->RU, out, lse, s);
  if (e != hipSuccess) return e;
  zha_time_end(t, s, ZHA_K_MERGE, 0);
  return hipSuccess;
}

hipError_t zha_launch_dense(const void* q, const void* K, const void* V, const ZLens& len, int B, int Hq, int Hkv,
                            int d, int64_t T, zha_dtype dt, float scale, float* out, float* lse, float* part, int WA,
                            hipStream_t s) {
  AttArgs a;
  a.q = q; a.K = K; a.V = V;
  a.kept = nullptr;
  a.kept_count = nullptr;
  a.cap1 = 0;
  a.part = part;
  a.W = WA;
  a.U = B * Hkv;
  a.hr = 1;
  a.Tq = 1;
  a.qtail = 0;
  a.Hkv = Hkv;
  a.Hq = Hq;
  a.G = Hq / Hkv;
  a.C = 1;
  a.Cshift = 0;
  a.T = T;
  a.scale_log2 = scale * ZHA_LOG2E;
  a.lens = nullptr;
  a.krank = nullptr;
  a.route_ctr = nullptr;
  a.ulist = nullptr;
  a.ucount = nullptr;
  a.TS = 0;
  a.NTC = 1;
  const int U = B * Hkv;
  LensArg<true> la;
  la.len = len;
  hipError_t e = launch_att_dt<true>(a, la, dt, d, U, s);
  if (e != hipSuccess) return e;
  return d == 64 ? launch_merge<64>(a, U, out, lse, s) : launch_merge<128>(a, U, out, lse, s);
}

__global__ void zha_copy16_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t n) {
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) dst[i] = src[i];
}

hipError_t zha_launch_copy16(void* dst, const void* src, int64_t n16, hipStream_t s) {
  hipLaunchKernelGGL(zha_copy16_kernel, dim3(2048), dim3(256), 0, s, (const uint4*)src, (uint4*)dst, n16);
  return hipGetLastError();
}
