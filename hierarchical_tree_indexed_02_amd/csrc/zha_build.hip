// zha_build.hip -- summary tree construction and incremental growth.
//
// Every node stores, per reference query r, the tangent plane of its log
// attention mass at q = r ([wqu] "Building the tree"; page key in include/zha.h):
//   LSE_r = log sum_{t in node} exp(r.k_t),  m_r = sum_t softmax_t(r.k) k_t,
//   b_r = LSE_r - r.m~_r  with m~_r the stored (rounded) m_r,
// so the plane b_r + q.m~_r is exact at q = r for the stored values.  Leaves
// cover C raw tokens; a parent is the exact log-sum-exp combination of its C
// children's fp32 (LSE, mean) ([aitop] abstract: recursively compressed key
// summaries).  The build runs in two kernels.  zha_build_subtree_kernel: one
// workgroup per node of the subtree level S (the highest level covering at most
// 256 tokens) streams that node's tokens in order, four tokens ahead of use:
// tokens fold into the leaf accumulator (registers), each finished leaf folds
// into its parent's accumulator (LDS), each finished node cascades upward, and
// a finished level-S node leaves its fp32 (LSE, mean) in a scratch buffer.
// zha_build_upper_kernel: one workgroup per top node folds those level-S
// results, in order, into levels S+1..L.  Every node folds the same values in
// the same order as a single pass over all levels would, so the split changes
// no bit of the result.  Thread (r, lane) owns reference query r and a 16th of
// the head dimension.
//
// Growth: the accumulators of each unit's rightmost open nodes (the "spine")
// are kept in fp32.  zha_append folds newly completed leaves into them with
// the same code in the same order, so the grown tree is bit-identical to a
// rebuild.  Open (partial) nodes are written by folding the partial child
// into a copy of the parent's accumulator, level by level.
#include "zha_internal.h"

namespace {

struct BuildArgs {
  const void* K;            // [B][Hkv][T][d]
  const float* refs;        // [Hkv][R][d]
  void* m[ZHA_MAX_LEVELS + 2];
  float* b[ZHA_MAX_LEVELS + 2];
  float* ms[ZHA_MAX_LEVELS + 2];    // fp8 summaries: row scales (m holds e4m3 codes); fp4: scale bytes per
                                    // block of 32 (m holds e2m1 codes); null entries otherwise
  int f4;                           // the low-precision summaries are fp4
  int64_t cap[ZHA_MAX_LEVELS + 2];
  int64_t lpn[ZHA_MAX_LEVELS + 2];  // leaves per node at level l: C^(l-1)
  float* spine;             // [U][L+1][E+2][NT]
  float* sub_lse;           // [U][cap_S][R] fp32 LSE of finished level-S nodes (null when S = L)
  float* sub_m;             // [U][cap_S][R][d] fp32 means of finished level-S nodes
  int S;                    // subtree level
  int L, C, R, Hkv;
  int Cshift;               // log2 C when C is a power of two, else -1
  int64_t T;
  ZLens len;                // lengths after the operation
  ZLens len_prev;           // append: lengths before it
  int32_t* geo;             // [L+2][B]: row 0 the lengths, row l the nodes of level l per sequence
  int B;
};

// Row 0 of the geometry table holds each sequence's length, row l (1..L) its number of
// level-l nodes, ceil(Nc / C^l) with Nc = C*floor(N / C); row L+1 is zero.  The routing
// kernels read their frontier sizes here instead of taking them by value.  Written by
// workgroup (0, 0) of the first kernel of a build or an append.
__device__ __forceinline__ void write_geo(const BuildArgs& a) {
  if (blockIdx.x != 0 || blockIdx.y != 0) return;
  for (int b = threadIdx.x; b < a.B; b += blockDim.x) {
    const int64_t N = a.len.n[b];
    const int64_t Nc = (N / a.C) * a.C;
    a.geo[b] = (int32_t)N;
    int64_t span = 1;
    for (int l = 1; l <= a.L; ++l) {
      span *= a.C;
      a.geo[(int64_t)l * a.B + b] = (int32_t)((Nc + span - 1) / span);
    }
    a.geo[(int64_t)(a.L + 1) * a.B + b] = 0;
  }
}

// Node indices fit in 32 bits (C^L <= 2^30 and max_tokens < 2^31): divisions by C are
// shifts when C is a power of two.
__device__ __forceinline__ int div_c(const BuildArgs& a, int x) { return a.Cshift >= 0 ? x >> a.Cshift : x / a.C; }
__device__ __forceinline__ bool last_child(const BuildArgs& a, int x) {
  return (a.Cshift >= 0 ? ((x + 1) & ((1 << a.Cshift) - 1)) : (x + 1) % a.C) == 0;
}

#pragma clang fp contract(off)

template <typename T, int E>
__device__ __forceinline__ void load_slice(const T* p, float (&k)[E]) {
#pragma unroll
  for (int e = 0; e < E; ++e) k[e] = Mf<T>::to_f32(p[e]);
}

template <int E>
__device__ __forceinline__ float dot_slice(const float (&a)[E], const float (&b)[E]) {
  float s = a[0] * b[0];
#pragma unroll
  for (int e = 1; e < E; ++e) s = __builtin_fmaf(a[e], b[e], s);
  return sum16(s);
}

// A leaf is accumulated in blocks of up to four consecutive tokens from its first token:
// the block's logits are independent, so they are formed together; the running
// (max, sum, weighted key sum) is rescaled once per block.  Build and append both
// accumulate leaves with this routine, so their planes agree bit for bit.
template <int E>
__device__ __forceinline__ void leaf_block_fold(Acc<E>& a, const float (&x)[4], const float (&k)[4][E], int n) {
  float bm = x[0];
#pragma unroll
  for (int i = 1; i < 4; ++i) bm = i < n ? fmaxf(bm, x[i]) : bm;
  const bool empty = a.S == 0.0f;
  const float nm = empty ? bm : fmaxf(a.M, bm);
  const float sc = empty ? 0.0f : zexp(a.M - nm);
  float w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = i < n ? zexp(x[i] - nm) : 0.0f;
  float S = a.S * sc;
#pragma unroll
  for (int i = 0; i < 4; ++i) S = S + w[i];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    float v = a.V[e] * sc;
#pragma unroll
    for (int i = 0; i < 4; ++i) v = __builtin_fmaf(w[i], k[i][e], v);
    a.V[e] = v;
  }
  a.M = nm;
  a.S = S;
}

// Folds a block of n <= 4 tokens (keys as stored) into a leaf accumulator.
template <typename T, int E>
__device__ __forceinline__ void leaf_block(Acc<E>& a, const float (&rv)[E], const T (&kb)[4][E], int n) {
  float k[4][E], x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int e = 0; e < E; ++e) k[i][e] = Mf<T>::to_f32(kb[i][e]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = dot_slice<E>(rv, k[i]);
  leaf_block_fold(a, x, k, n);
}

// Keys of tokens [t, t + 4) clamped to t_last (the block's valid count is passed apart).
template <typename T, int E, int D>
__device__ __forceinline__ void load_block(const T* Kb, int64_t t, int64_t t_last, int ln, T (&kb)[4][E]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t tt = min(t + i, t_last);
#pragma unroll
    for (int e = 0; e < E; ++e) kb[i][e] = Kb[tt * D + ln * E + e];
  }
}

// (LSE, mean slice) of leaf chunk c of this unit from its C raw keys.
template <typename T, int E, int D>
__device__ __forceinline__ void leaf_planes(const T* Kb, int64_t c, int C, int ln, const float (&rv)[E], float& lse,
                                            float (&m)[E]) {
  Acc<E> acc;
  acc_clear(acc);
  for (int b = 0; b < C; b += 4) {
    T kb[4][E];
    load_block<T, E, D>(Kb, c * C + b, c * C + C - 1, ln, kb);
    leaf_block<T, E>(acc, rv, kb, min(4, C - b));
  }
  acc_finish(acc, lse, m);
}

// fp4 codes of one lane's E values (scaled by 2^-ex, |value| <= 6 after scaling), element 2i
// in the low nibble of byte i, and the decoded values m~ = code * 2^ex.
template <int E>
__device__ __forceinline__ uint32_t fp4_encode(const float (&m)[E], int ex, float (&mt)[E]) {
  static_assert(E == 4 || E == 8, "two or four code bytes per lane");
  float x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = __builtin_ldexpf(m[e], -ex);
  const float sc = __builtin_ldexpf(1.0f, ex);
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x[0], x[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[2], x[3], 1.0f, 1);
  auto v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 0);
  auto v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 1);
  mt[0] = v0[0]; mt[1] = v0[1]; mt[2] = v1[0]; mt[3] = v1[1];
  if constexpr (E == 8) {
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[4], x[5], 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[6], x[7], 1.0f, 3);
    auto v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 2);
    auto v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 3);
    mt[4] = v2[0]; mt[5] = v2[1]; mt[6] = v3[0]; mt[7] = v3[1];
  }
  return w;
}

// Store node j of level l: m~ = m rounded to the storage type, b = LSE - r.m~.  With fp8
// summaries the row (16 lanes) shares one power-of-two scale from its largest magnitude;
// with fp4, each block of 32 values (32/E lanes) has its own.
template <typename T, int E, int D>
__device__ __forceinline__ void emit(const BuildArgs& a, int u, int l, int64_t j, int r, int ln, const float (&rv)[E],
                                     float lse, const float (&m)[E]) {
  const int64_t row = ((int64_t)u * a.cap[l] + j) * a.R + r;
  float mt[E];
  if (a.ms[l] && a.f4) {
    constexpr int LB = 32 / E;  // lanes per block: a quad (d = 128) or a half row (d = 64)
    static_assert(LB == 4 || LB == 8, "blocks of 32 values");
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(m[e]));
    amax = fmaxf(amax, dpp_mov<0xB1>(amax));   // quad_perm [1,0,3,2]
    amax = fmaxf(amax, dpp_mov<0x4E>(amax));   // quad_perm [2,3,0,1]: the quad's maximum
    if (LB == 8) amax = fmaxf(amax, dpp_mov<0x141>(amax));  // row_half_mirror: the half row's
    const int ex = fp4_block_exp(amax);
    const uint32_t w = fp4_encode<E>(m, ex, mt);
    uint8_t* cp = (uint8_t*)a.m[l] + row * (D / 2) + ln * (E / 2);
    if constexpr (E == 8) *(uint32_t*)cp = w;
    else *(uint16_t*)cp = (uint16_t)w;
    if (ln % LB == 0) ((uint8_t*)a.ms[l])[row * (D / 32) + ln / LB] = (uint8_t)(ex + 127);
  } else if (a.ms[l]) {
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(m[e]));
    const int ex = fp8_row_exp(max16(amax));
    static_assert(E % 4 == 0, "whole code words per lane");
    uint32_t* cp = (uint32_t*)((uint8_t*)a.m[l] + row * D + ln * E);
#pragma unroll
    for (int i = 0; i < E / 4; ++i) {
      // hardware conversions: round to nearest even onto the e4m3 grid (|x| <= 448 here),
      // and back (exact)
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_ldexpf(m[4 * i], -ex), __builtin_ldexpf(m[4 * i + 1], -ex), 0,
                                              false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_ldexpf(m[4 * i + 2], -ex), __builtin_ldexpf(m[4 * i + 3], -ex), w,
                                          true);
      cp[i] = (uint32_t)w;
      const auto v01 = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
      const auto v23 = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
      mt[4 * i] = __builtin_ldexpf(v01[0], ex);
      mt[4 * i + 1] = __builtin_ldexpf(v01[1], ex);
      mt[4 * i + 2] = __builtin_ldexpf(v23[0], ex);
      mt[4 * i + 3] = __builtin_ldexpf(v23[1], ex);
    }
    if (ln == 0) a.ms[l][row] = __builtin_ldexpf(1.0f, ex);
  } else {
    T* mp = (T*)a.m[l] + row * D + ln * E;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const T x = Mf<T>::from_f32(m[e]);
      mp[e] = x;
      mt[e] = Mf<T>::to_f32(x);
    }
  }
  const float rm = dot_slice<E>(rv, mt);
  if (ln == 0) a.b[l][row] = lse - rm;
}

// Accumulator stack of levels lbase.. in LDS, struct-of-arrays [l - lbase][E+2][NT].
template <int E> struct Stack {
  float* base;
  int NT, tid, lbase;
  __device__ float& M(int l) { return base[((int64_t)(l - lbase) * (E + 2) + 0) * NT + tid]; }
  __device__ float& S(int l) { return base[((int64_t)(l - lbase) * (E + 2) + 1) * NT + tid]; }
  __device__ float& V(int l, int e) { return base[((int64_t)(l - lbase) * (E + 2) + 2 + e) * NT + tid]; }
  __device__ void get(int l, Acc<E>& a) {
    a.M = M(l); a.S = S(l);
#pragma unroll
    for (int e = 0; e < E; ++e) a.V[e] = V(l, e);
  }
  __device__ void put(int l, const Acc<E>& a) {
    M(l) = a.M; S(l) = a.S;
#pragma unroll
    for (int e = 0; e < E; ++e) V(l, e) = a.V[e];
  }
};

template <int E, int D>
__device__ __forceinline__ void put_sub(const BuildArgs& a, int u, int64_t j, int r, int ln, float lse,
                                        const float (&m)[E]) {
  float* mp = a.sub_m + (((int64_t)u * a.cap[a.S] + j) * a.R + r) * D + ln * E;
#pragma unroll
  for (int e = 0; e < E; ++e) mp[e] = m[e];
  if (ln == 0) a.sub_lse[((int64_t)u * a.cap[a.S] + j) * a.R + r] = lse;
}

template <int E, int D>
__device__ __forceinline__ void get_sub(const BuildArgs& a, int u, int64_t j, int r, int ln, float& lse,
                                        float (&m)[E]) {
  const float* mp = a.sub_m + (((int64_t)u * a.cap[a.S] + j) * a.R + r) * D + ln * E;
#pragma unroll
  for (int e = 0; e < E; ++e) m[e] = mp[e];
  lse = a.sub_lse[((int64_t)u * a.cap[a.S] + j) * a.R + r];
}

// Finished node j of level l0 (its planes already stored): fold it into its ancestors up
// to level ltop, finishing and storing every ancestor whose last child it is.  A finished
// node of level ltop is handed back (returns true) instead of folding further.
template <typename T, int E, int D>
__device__ __forceinline__ bool push_node(const BuildArgs& a, Stack<E>& st, int u, int l0, int j, int ltop,
                                          int r, int ln, const float (&rv)[E], float& lse, float (&m)[E]) {
  int idx = j;  // index of the finished node at the current level
  for (int l = l0 + 1; l <= ltop; ++l) {
    Acc<E> acc;
    st.get(l, acc);
    acc_fold(acc, lse, m);
    if (!last_child(a, idx)) {
      st.put(l, acc);
      return false;
    }
    idx = div_c(a, idx);
    acc_finish(acc, lse, m);
    emit<T, E, D>(a, u, l, idx, r, ln, rv, lse, m);
    acc_clear(acc);
    st.put(l, acc);
  }
  return true;
}

// Writes the open (partial) node of levels l0..l1 for a unit with n1 leaves: each open
// node is its accumulator (complete children only) with the open child below folded in.
// (carry, clse, cm) is the open child of level l0 on entry and the open node of level l1
// on return.
template <typename T, int E, int D>
__device__ __forceinline__ void flush_open(const BuildArgs& a, Stack<E>& st, int u, int64_t n1, int l0, int l1, int r,
                                           int ln, const float (&rv)[E], bool& carry, float& clse, float (&cm)[E]) {
  for (int l = l0; l <= l1; ++l) {
    if (n1 % a.lpn[l] == 0) { carry = false; continue; }
    Acc<E> acc;
    st.get(l, acc);
    if (carry) acc_fold(acc, clse, cm);
    acc_finish(acc, clse, cm);
    emit<T, E, D>(a, u, l, (n1 - 1) / a.lpn[l], r, ln, rv, clse, cm);
    carry = true;
  }
}

template <int E>
__device__ __forceinline__ void stack_clear(Stack<E>& st, int l0, int l1) {
  for (int l = l0; l <= l1; ++l) {
    Acc<E> z;
    acc_clear(z);
    st.put(l, z);
  }
}

template <int E>
__device__ __forceinline__ void spine_io(const BuildArgs& a, Stack<E>& st, int u, int l0, int l1, bool store) {
  float* sp = a.spine + (int64_t)u * (a.L + 1) * (E + 2) * st.NT;
  for (int l = l0; l <= l1; ++l)
    for (int f = 0; f < E + 2; ++f) {
      float* g = sp + ((int64_t)l * (E + 2) + f) * st.NT + st.tid;
      float* s = st.base + ((int64_t)(l - st.lbase) * (E + 2) + f) * st.NT + st.tid;
      if (store) *g = *s; else *s = *g;
    }
}

// One workgroup per (level-S node, unit); blockDim = 16 R.
template <typename T, int D>
__global__ __launch_bounds__(256, 4) void zha_build_subtree_kernel(BuildArgs a) {
  write_geo(a);
  constexpr int E = D / 16;
  extern __shared__ float lds[];
  const int NT = blockDim.x;
  const int tid = threadIdx.x, r = tid >> 4, ln = tid & 15;
  const int u = blockIdx.y, bi = u / a.Hkv, g = u % a.Hkv;
  const int64_t N = a.len.n[bi];
  const int n1 = (int)(N / a.C);
  const int S = a.S;
  const int per = (int)a.lpn[S];  // leaves per level-S node
  const int j = blockIdx.x;
  const int c0 = j * per;
  Stack<E> st{lds, NT, tid, 2};
  if (c0 >= n1) {
    if (j == 0) {  // no complete leaf: the unit has an empty spine
      stack_clear(st, 2, S);
      spine_io(a, st, u, 2, S, true);
    }
    return;
  }
  const int c1 = min(c0 + per, n1);
  float rv[E];
  load_slice<float, E>(a.refs + ((int64_t)g * a.R + r) * D + ln * E, rv);
  const T* Kb = (const T*)a.K + ((int64_t)bi * a.Hkv + g) * a.T * D;
  stack_clear(st, 2, S);
  // leaves [c0, c1) in order, each in blocks of four tokens from its first token; the
  // keys of the next block are loaded while the current one is folded
  T kA[4][E], kB[4][E];
  Acc<E> leaf;
  acc_clear(leaf);
  int qc = c0, qb = 0;  // block being loaded next: leaf qc, tokens qb..qb+3
  auto fetch = [&](T (&kb)[4][E]) {
    if (qc >= c1) return;
    load_block<T, E, D>(Kb, (int64_t)qc * a.C + qb, (int64_t)qc * a.C + a.C - 1, ln, kb);
    qb += 4;
    if (qb >= a.C) { qb = 0; ++qc; }
  };
  int cc = c0, cb = 0;  // block being folded: leaf cc, tokens cb..cb+3
  auto consume = [&](const T (&kb)[4][E]) {
    leaf_block<T, E>(leaf, rv, kb, min(4, a.C - cb));
    cb += 4;
    if (cb >= a.C) {  // the leaf's last block
      float lse, m[E];
      acc_finish(leaf, lse, m);
      acc_clear(leaf);
      emit<T, E, D>(a, u, 1, cc, r, ln, rv, lse, m);
      if (push_node<T, E, D>(a, st, u, 1, cc, S, r, ln, rv, lse, m) && a.sub_m)
        put_sub<E, D>(a, u, j, r, ln, lse, m);
      cb = 0;
      ++cc;
    }
  };
  fetch(kA);
  while (cc < c1) {
    fetch(kB);
    consume(kA);
    if (cc >= c1) break;
    fetch(kA);
    consume(kB);
  }
  if (c1 == n1) {  // the unit's last level-S node: keep its open accumulators, write its open nodes
    spine_io(a, st, u, 2, S, true);
    bool carry = false;
    float clse = 0.0f, cm[E];
#pragma unroll
    for (int e = 0; e < E; ++e) cm[e] = 0.0f;
    flush_open<T, E, D>(a, st, u, n1, 2, S, r, ln, rv, carry, clse, cm);
    if (carry && a.sub_m) put_sub<E, D>(a, u, j, r, ln, clse, cm);  // the open level-S node
  }
}

// One workgroup per (top node, unit): levels S+1..L from the finished level-S nodes.
template <typename T, int D>
__global__ __launch_bounds__(256) void zha_build_upper_kernel(BuildArgs a) {
  constexpr int E = D / 16;
  extern __shared__ float lds_stack[];
  const int tid = threadIdx.x, r = tid >> 4, ln = tid & 15;
  const int u = blockIdx.y, g = u % a.Hkv;
  const int64_t n1 = a.len.n[u / a.Hkv] / a.C;
  const int S = a.S;
  const int64_t perS = a.lpn[S];
  const int64_t nS_done = n1 / perS, nS_all = (n1 + perS - 1) / perS;
  const int64_t cpt = a.lpn[a.L] / perS;  // level-S nodes per top node
  const int64_t T0 = blockIdx.x;
  const int64_t j0 = T0 * cpt;
  Stack<E> st{lds_stack, (int)blockDim.x, tid, S + 1};
  if (j0 >= nS_all) {
    if (T0 == 0) {
      stack_clear(st, S + 1, a.L);
      spine_io(a, st, u, S + 1, a.L, true);
    }
    return;
  }
  float rv[E];
  load_slice<float, E>(a.refs + ((int64_t)g * a.R + r) * D + ln * E, rv);
  stack_clear(st, S + 1, a.L);
  const int64_t j1 = min(j0 + cpt, nS_done);
  float lse, m[E];
  if (j0 < j1) get_sub<E, D>(a, u, j0, r, ln, lse, m);
  for (int64_t jj = j0; jj < j1; ++jj) {
    float nlse = 0.0f, nm[E];
    if (jj + 1 < j1) get_sub<E, D>(a, u, jj + 1, r, ln, nlse, nm);  // next child in flight
    push_node<T, E, D>(a, st, u, S, (int)jj, a.L, r, ln, rv, lse, m);
    lse = nlse;
#pragma unroll
    for (int e = 0; e < E; ++e) m[e] = nm[e];
  }
  if (j0 + cpt >= nS_all) {  // the unit's last top node
    spine_io(a, st, u, S + 1, a.L, true);
    bool carry = n1 % perS != 0;  // the open level-S node, written by the subtree kernel
    float clse = 0.0f, cm[E];
#pragma unroll
    for (int e = 0; e < E; ++e) cm[e] = 0.0f;
    if (carry) get_sub<E, D>(a, u, nS_all - 1, r, ln, clse, cm);
    flush_open<T, E, D>(a, st, u, n1, S + 1, a.L, r, ln, rv, carry, clse, cm);
  }
}

// One workgroup per unit: fold the leaves completed by the new rows through every level.
template <typename T, int D>
__global__ __launch_bounds__(256) void zha_append_kernel(BuildArgs a) {
  write_geo(a);
  constexpr int E = D / 16;
  extern __shared__ float lds_stack[];
  const int tid = threadIdx.x, r = tid >> 4, ln = tid & 15;
  const int u = blockIdx.x, bi = u / a.Hkv, g = u % a.Hkv;
  const int64_t n1_old = a.len_prev.n[bi] / a.C;
  const int64_t n1 = a.len.n[bi] / a.C;
  if (n1 == n1_old) return;
  Stack<E> st{lds_stack, (int)blockDim.x, tid, 2};
  float rv[E];
  load_slice<float, E>(a.refs + ((int64_t)g * a.R + r) * D + ln * E, rv);
  const T* Kb = (const T*)a.K + ((int64_t)bi * a.Hkv + g) * a.T * D;
  spine_io(a, st, u, 2, a.L, false);
  for (int64_t c = n1_old; c < n1; ++c) {
    float lse, m[E];
    leaf_planes<T, E, D>(Kb, c, a.C, ln, rv, lse, m);
    emit<T, E, D>(a, u, 1, c, r, ln, rv, lse, m);
    push_node<T, E, D>(a, st, u, 1, (int)c, a.L, r, ln, rv, lse, m);
  }
  spine_io(a, st, u, 2, a.L, true);
  bool carry = false;
  float clse = 0.0f, cm[E];
#pragma unroll
  for (int e = 0; e < E; ++e) cm[e] = 0.0f;
  flush_open<T, E, D>(a, st, u, n1, 2, a.L, r, ln, rv, carry, clse, cm);
}

#pragma clang fp contract(on)

BuildArgs make_args(const zha_tree* t, const void* K) {
  BuildArgs a;
  a.K = K;
  a.refs = t->refs;
  for (int l = 0; l < ZHA_MAX_LEVELS + 2; ++l) {
    a.m[l] = t->m[l];
    a.b[l] = t->b[l];
    a.ms[l] = t->ms[l];
    a.f4 = t->f4 ? 1 : 0;
    a.cap[l] = t->cap[l];
    a.lpn[l] = l >= 1 ? t->span[l] / t->C : 1;
  }
  a.spine = t->spine;
  a.sub_lse = t->sub_lse;
  a.sub_m = t->sub_m;
  a.S = t->S;
  a.Cshift = -1;
  for (int sh = 0; sh < 31; ++sh)
    if ((1 << sh) == t->C) a.Cshift = sh;
  a.L = t->L;
  a.C = t->C;
  a.R = t->R;
  a.Hkv = t->desc.n_kv_heads;
  a.T = t->T;
  a.len = t->len;
  a.len_prev = t->len_prev;
  a.geo = t->geo;
  a.B = t->desc.batch;
  return a;
}

// Decoded fp8 summaries: out[row][k] = value(code[row][k]) * scale[row], exact in bf16.
__global__ __launch_bounds__(256) void zha_decode_fp8_kernel(const uint8_t* codes, const float* scale, int64_t rows,
                                                              int d, __bf16* out) {
  const int64_t n = rows * d;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float v = fp8_value(codes[i]) * scale[i / d];
    out[i] = Mf<__bf16>::from_f32(v);
  }
}

}  // namespace

// LDS accumulator stack of nlev levels; the spine in HBM keeps levels 0..L (0 and 1 unused).
size_t zha_stack_bytes(int nlev, int d, int R) {
  return (size_t)(nlev > 0 ? nlev : 0) * (d / 16 + 2) * (16 * R) * sizeof(float);
}

size_t zha_spine_bytes(int L, int d, int R) { return zha_stack_bytes(L + 1, d, R); }

// Largest dynamic LDS any build kernel asks for.
size_t zha_build_lds_bytes(int S, int L, int d, int R, int esize) {
  (void)esize;
  size_t m = zha_stack_bytes(S - 1, d, R);                         // subtree
  if (zha_stack_bytes(L - S, d, R) > m) m = zha_stack_bytes(L - S, d, R);  // upper
  if (zha_stack_bytes(L - 1, d, R) > m) m = zha_stack_bytes(L - 1, d, R);  // append
  return m;
}

// Kernels whose accumulator stack exceeds the default dynamic LDS limit opt in to more.
template <typename F>
hipError_t allow_lds(F kernel, size_t bytes) {
  return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <typename T, int D>
hipError_t launch_build_td(zha_tree* t, const BuildArgs& a, hipStream_t s) {
  const size_t sh_sub = zha_stack_bytes(t->S - 1, t->d, t->R);
  const size_t sh_up = zha_stack_bytes(t->L - t->S, t->d, t->R);
  hipError_t e = allow_lds(zha_build_subtree_kernel<T, D>, sh_sub);
  if (e != hipSuccess) return e;
  dim3 block(16 * t->R);
  zha_time_begin(t, s, ZHA_K_BUILD, t->S);
  hipLaunchKernelGGL((zha_build_subtree_kernel<T, D>), dim3((unsigned)(t->cap[t->S] > 0 ? t->cap[t->S] : 1), (unsigned)t->U),
                     block, sh_sub, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  zha_time_end(t, s, ZHA_K_BUILD, t->S);
  if (t->S == t->L) return hipSuccess;
  e = allow_lds(zha_build_upper_kernel<T, D>, sh_up);
  if (e != hipSuccess) return e;
  zha_time_begin(t, s, ZHA_K_BUILD, t->L);
  hipLaunchKernelGGL((zha_build_upper_kernel<T, D>), dim3((unsigned)(t->cap[t->L] > 0 ? t->cap[t->L] : 1), (unsigned)t->U),
                     block, sh_up, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  zha_time_end(t, s, ZHA_K_BUILD, t->L);
  return hipSuccess;
}

// The subtree kernel is timed as build level S, the upper kernel as build level L.
hipError_t zha_launch_build(zha_tree* t, const void* K, hipStream_t s) {
  BuildArgs a = make_args(t, K);
  if (t->desc.dtype == ZHA_BF16)
    return t->d == 64 ? launch_build_td<__bf16, 64>(t, a, s) : launch_build_td<__bf16, 128>(t, a, s);
  return t->d == 64 ? launch_build_td<float, 64>(t, a, s) : launch_build_td<float, 128>(t, a, s);
}

hipError_t zha_launch_append(zha_tree* t, const void* K, hipStream_t s) {
  BuildArgs a = make_args(t, K);
  const size_t sh = zha_stack_bytes(t->L - 1, t->d, t->R);
  hipError_t e0 = t->desc.dtype == ZHA_BF16
                      ? (t->d == 64 ? allow_lds(zha_append_kernel<__bf16, 64>, sh) : allow_lds(zha_append_kernel<__bf16, 128>, sh))
                      : (t->d == 64 ? allow_lds(zha_append_kernel<float, 64>, sh) : allow_lds(zha_append_kernel<float, 128>, sh));
  if (e0 != hipSuccess) return e0;
  dim3 grid((unsigned)t->U), block(16 * t->R);
  zha_time_begin(t, s, ZHA_K_APPEND, 0);
  if (t->desc.dtype == ZHA_BF16) {
    if (t->d == 64) hipLaunchKernelGGL((zha_append_kernel<__bf16, 64>), grid, block, sh, s, a);
    else hipLaunchKernelGGL((zha_append_kernel<__bf16, 128>), grid, block, sh, s, a);
  } else {
    if (t->d == 64) hipLaunchKernelGGL((zha_append_kernel<float, 64>), grid, block, sh, s, a);
    else hipLaunchKernelGGL((zha_append_kernel<float, 128>), grid, block, sh, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  zha_time_end(t, s, ZHA_K_APPEND, 0);
  return hipSuccess;
}

// Decoded fp4 summaries: out[row][k] = value(code) * 2^e of k's block, exact in bf16, and the
// block scales as floats into scale_out [rows][d/32] (either output may be null).
__global__ __launch_bounds__(256) void zha_decode_fp4_kernel(const uint8_t* codes, const uint8_t* scale, int64_t rows,
                                                              int d, __bf16* out, float* scale_out) {
  const int64_t n = rows * d / 2;  // code bytes
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t k = (2 * i) % d, rw = (2 * i) / d;
    const float sc = fp4_scale(scale[rw * (d / 32) + k / 32]);
    if (out) {
      const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((uint32_t)codes[i], sc, 0);
      out[2 * i] = Mf<__bf16>::from_f32(v[0]);
      out[2 * i + 1] = Mf<__bf16>::from_f32(v[1]);
    }
    if (scale_out && k % 32 == 0) scale_out[rw * (d / 32) + k / 32] = sc;
  }
}

hipError_t zha_launch_decode_fp4(const uint8_t* codes, const uint8_t* scale, int64_t rows, int d, __bf16* out,
                                 float* scale_out, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  int64_t blocks = (rows * d / 2 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(zha_decode_fp4_kernel, dim3((unsigned)blocks), dim3(256), 0, s, codes, scale, rows, d, out,
                     scale_out);
  return hipGetLastError();
}

hipError_t zha_launch_decode_fp8(const uint8_t* codes, const float* scale, int64_t rows, int d, __bf16* out,
                                 hipStream_t s) {
  int64_t blocks = (rows * d + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(zha_decode_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, s, codes, scale, rows, d, out);
  return hipGetLastError();
}
