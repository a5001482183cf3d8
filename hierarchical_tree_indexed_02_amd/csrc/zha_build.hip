// zha_build.hip -- summary tree construction and incremental growth.
//
// Every node stores, per reference query r, the tangent plane of its log
// attention mass at q = r ([wqu] "Building the tree"; page key in include/zha.h):
//   LSE_r = log sum_{t in node} exp(r.k_t),  m_r = sum_t softmax_t(r.k) k_t,
//   b_r = LSE_r - r.m~_r  with m~_r the stored (rounded) m_r,
// so the plane b_r + q.m~_r is exact at q = r for the stored values.  Leaves
// cover C raw tokens; a parent is the exact log-sum-exp combination of its C
// children's fp32 (LSE, mean) ([aitop] abstract: recursively compressed key
// summaries).  Trees of bf16 keys with C = 4 are built by the matrix-core kernels of
// the section below (zha_build_c4_kernel and its upper-level and append kernels); every
// other tree by the per-thread kernels described here, in two kernels.
// zha_build_subtree_kernel: one
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
// with fp4, each block of 32 values (32/E lanes) has its own.  SF fixes the storage format at
// compile time (0 native, 1 fp8, 2 fp4); -1 reads it from the tree.
template <typename T, int E, int D, int SF = -1>
__device__ __forceinline__ void emit(const BuildArgs& a, int u, int l, int64_t j, int r, int ln, const float (&rv)[E],
                                     float lse, const float (&m)[E]) {
  const int64_t row = ((int64_t)u * a.cap[l] + j) * a.R + r;
  float mt[E];
  if (SF == 2 || (SF == -1 && a.ms[l] && a.f4)) {
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
  } else if (SF == 1 || (SF == -1 && a.ms[l])) {
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

// ======================================================================= matrix-core path (C = 4, bf16 keys)
//
// The same tree, computed with the matrix cores where the work is a dense product.  One wave
// holds a whole node: lane (g, c) = (lane / 16, lane % 16) holds reference rows r = 4 g + v
// (v = 0..3) and elements e = E c + b (b = 0..E-1), which is the output layout of a 16x16
// MFMA with rows r and columns c.  Rows r >= R are zero references whose results are never
// stored.  A tile of 16 consecutive tokens (four leaves, one level-2 node) is processed at
// once:
//   logits  X[t][r] = k_t . r_r on v_mfma_f32_16x16x32_bf16 (keys as the A operand, tokens as
//           rows).  The fp32 reference is split into three bf16 parts hi + mid + lo equal to it
//           exactly, so every product is exact and the sums are fp32.  Lane (g, c) ends with
//           the four logits of leaf g for reference c, so the leaf's maximum, exponentials,
//           sum and LSE are lane-local;
//   means   softmax weights pass through LDS into the operand layout of v_mfma_f32_16x16x4f32,
//           whose k = 4 is one leaf's four tokens: one instruction forms sum_t w_t k_t for 16
//           references x 16 elements.  A leaf takes E instructions; the level-2 node takes 4 E,
//           accumulating its four leaves' tokens with weights normalised over all sixteen;
//   levels >= 3  the exact log-sum-exp fold of each child (fold_row), per (r, e).
// Leaves and level-2 nodes are thus computed from their tokens by the definition ([wqu]
// "Building the tree"); higher levels combine children ([aitop] abstract), which gives the same
// value up to rounding.  A workgroup of four waves owns a level-4 node (64 leaves): wave w
// builds level-3 node 4 j + w, wave 0 folds the four into level 4.  Levels above 4 are folded
// by a workgroup per top node, one reference row per thread.  Growth (zha_append) computes
// each new leaf, and each level-2 node a new leaf completes or leaves open, with the same tile
// routine, and folds the higher levels with the same code, so an appended tree equals a
// rebuild bit for bit.

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
template <int E> struct KwVec;
template <> struct KwVec<8> { typedef bf16x8_t type; };
template <> struct KwVec<4> { typedef bf16x4_t type; };

// Per-wave exchange area (floats): leaf weights [16][20] (rows padded against bank conflicts),
// level-2 weights [16][20], leaf LSE [4][16], level-2 LSE [16].
constexpr int C4_WT = 20;
constexpr int C4_W2 = 16 * C4_WT;
constexpr int C4_L1 = 2 * 16 * C4_WT;
constexpr int C4_L2 = C4_L1 + 64;
constexpr int C4_WS = C4_L2 + 16;
// Per-wave slot of the workgroup kernel: the level-3 accumulator record while the wave's
// tiles run, then its finished (or open) level-3 node, LSE [16] and mean [16][D].
constexpr int c4_slot_floats(int D) { return 16 + 16 * D > (2 + D / 16) * 256 ? 16 + 16 * D : (2 + D / 16) * 256; }

// Keys of one tile for one lane: the logit operand (token row c, elements (D/4) g + 8 s ..
// + 8 for k-step s) and the mean operand of each leaf q (token row 4 q + g, elements E c ..
// E c + E).  Rows past the last complete leaf are clamped to it.
template <int D> struct Tile4 {
  bf16x8_t kl[D / 32];
  typename KwVec<D / 16>::type kw[4];
};

template <int D>
__device__ __forceinline__ void load_tile4(const __bf16* Kb, int64_t t0, int64_t tlast, int g, int c, Tile4<D>& tk) {
  constexpr int E = D / 16;
  const __bf16* pl = Kb + min(t0 + c, tlast) * D + (D / 4) * g;
#pragma unroll
  for (int s = 0; s < D / 32; ++s) tk.kl[s] = *(const bf16x8_t*)(pl + 8 * s);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    tk.kw[q] = *(const typename KwVec<E>::type*)(Kb + min(t0 + 4 * q + g, tlast) * D + E * c);
}

// The three bf16 parts of reference rows 0..15 of head gh in LDS, [part][r][D + 8] (rows
// padded by 16 bytes), and the rows themselves in fp32, rfl [r][D] (for b = LSE - r.m~); zero
// rows for r >= R.  Threads tid, tid + nt, ... of the workgroup.
template <int D>
__device__ __forceinline__ void refs_split(const BuildArgs& a, int gh, __bf16* rsl, float* rfl, int tid, int nt) {
  constexpr int RST = D + 8;
  for (int i = tid; i < 16 * D; i += nt) {
    const int r = i / D, k = i - r * D;
    const float x = r < a.R ? a.refs[((int64_t)gh * a.R + r) * D + k] : 0.0f;
    const __bf16 hi = Mf<__bf16>::from_f32(x);
    const float x1 = x - Mf<__bf16>::to_f32(hi);
    const __bf16 mid = Mf<__bf16>::from_f32(x1);
    const __bf16 lo = Mf<__bf16>::from_f32(x1 - Mf<__bf16>::to_f32(mid));
    rsl[r * RST + k] = hi;
    rsl[(16 + r) * RST + k] = mid;
    rsl[(32 + r) * RST + k] = lo;
    rfl[i] = x;
  }
}

// Orders this wave's LDS accesses (LDS executes one wave's instructions in order; this keeps
// the compiler from moving them across).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Maximum / sum over the four rows of 16 lanes (lanes c, 16 + c, 32 + c, 48 + c), the same
// bits in all four.
__device__ __forceinline__ float rows4_max(float x) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float rows4_sum(float x) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Logits of a tile and its softmax weights, into the wave's exchange area ws: for leaf g and
// reference c, the weights of tokens 4 g + v normalised over the leaf (ws[c][4 g + v]) and the
// leaf's LSE (ws[C4_L1 + 16 g + c]).  With lvl2, also the weights normalised over the level-2
// node made of the tile's first nl complete leaves (ws[C4_W2 + c][4 g + v], zero for tokens of
// later leaves) and its LSE (ws[C4_L2 + c]).
template <int D>
__device__ __forceinline__ void tile_weights(const Tile4<D>& tk, const __bf16* rsl, int g, int c, int nl, bool lvl2,
                                             float* ws) {
  constexpr int RST = D + 8;
  f32x4_t x[3];
#pragma unroll
  for (int p = 0; p < 3; ++p) x[p] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < D / 32; ++s)
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      const bf16x8_t rb = *(const bf16x8_t*)(rsl + (p * 16 + c) * RST + (D / 4) * g + 8 * s);
      x[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tk.kl[s], rb, x[p], 0, 0, 0);
    }
  float X[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) X[v] = (x[2][v] + x[1][v]) + x[0][v];
  const float mx = fmaxf(fmaxf(X[0], X[1]), fmaxf(X[2], X[3]));
  float w[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) w[v] = zexp(X[v] - mx);
  const float s = ((w[0] + w[1]) + w[2]) + w[3];
  const float lse = mx + zlog(s);
  const float inv = __builtin_amdgcn_rcpf(s);
  *(float4*)(ws + c * C4_WT + 4 * g) = make_float4(w[0] * inv, w[1] * inv, w[2] * inv, w[3] * inv);
  ws[C4_L1 + g * 16 + c] = lse;
  if (lvl2) {
    const bool in = g < nl;
    const float lv = in ? lse : -INFINITY;
    const float M2 = rows4_max(lv);
    const float S2 = rows4_sum(zexp(lv - M2));
    const float lse2 = M2 + zlog(S2);
    float w2[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) w2[v] = in ? zexp(X[v] - lse2) : 0.0f;
    *(float4*)(ws + C4_W2 + c * C4_WT + 4 * g) = make_float4(w2[0], w2[1], w2[2], w2[3]);
    if (g == 0) ws[C4_L2 + c] = lse2;
  }
  wave_lds_sync();
}

// fp32 values of the mean operand of leaf q.
template <int E>
__device__ __forceinline__ void kw_f32(const typename KwVec<E>::type& kw, float (&k)[E]) {
#pragma unroll
  for (int b = 0; b < E; ++b) k[b] = (float)kw[b];
}

// Leaf q of the tile in node layout (kwq = the tile's kw[q]): LSE of rows 4 g + v and mean
// elements E c + b.
template <int D>
__device__ __forceinline__ void leaf_mean4(const typename KwVec<D / 16>::type& kwq, int q, int g, int c, const float* ws,
                                           float (&lse)[4], float (&m)[4][D / 16]) {
  constexpr int E = D / 16;
  const float aq = ws[c * C4_WT + 4 * q + g];
  const float4 lq = *(const float4*)(ws + C4_L1 + q * 16 + 4 * g);
  lse[0] = lq.x; lse[1] = lq.y; lse[2] = lq.z; lse[3] = lq.w;
  float k[E];
  kw_f32<E>(kwq, k);
  const f32x4_t z = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int b = 0; b < E; ++b) {
    const f32x4_t d = __builtin_amdgcn_mfma_f32_16x16x4f32(aq, k[b], z, 0, 0, 0);
#pragma unroll
    for (int v = 0; v < 4; ++v) m[v][b] = d[v];
  }
}

// The tile's level-2 node (as tile_weights with lvl2) in node layout.
template <int D>
__device__ __forceinline__ void level2_mean4(const Tile4<D>& tk, int g, int c, const float* ws, float (&lse)[4],
                                             float (&m)[4][D / 16]) {
  constexpr int E = D / 16;
  const float4 l2 = *(const float4*)(ws + C4_L2 + 4 * g);
  lse[0] = l2.x; lse[1] = l2.y; lse[2] = l2.z; lse[3] = l2.w;
  f32x4_t acc[E];
#pragma unroll
  for (int b = 0; b < E; ++b) acc[b] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float aq = ws[C4_W2 + c * C4_WT + 4 * q + g];
    float k[E];
    kw_f32<E>(tk.kw[q], k);
#pragma unroll
    for (int b = 0; b < E; ++b) acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(aq, k[b], acc[b], 0, 0, 0);
  }
#pragma unroll
  for (int b = 0; b < E; ++b)
#pragma unroll
    for (int v = 0; v < 4; ++v) m[v][b] = acc[b][v];
}

// Exact log-sum-exp fold of child (x, m) into accumulator a, without branches: with d = x - M,
// the smaller side is scaled by exp(-|d|).  An empty accumulator (M = -inf, S = 0, V = 0)
// takes the child exactly.
template <int E> __device__ __forceinline__ void fold_row(Acc<E>& a, float x, const float (&m)[E]) {
  const float d = x - a.M;
  const bool up = d > 0.0f;
  const float ce = zexp(up ? -d : d);
  const float co = up ? ce : 1.0f, cn = up ? 1.0f : ce;
  a.S = __builtin_fmaf(a.S, co, cn);
#pragma unroll
  for (int e = 0; e < E; ++e) a.V[e] = __builtin_fmaf(cn, m[e], a.V[e] * co);
  a.M = up ? x : a.M;
}
template <int E> __device__ __forceinline__ void finish_row(const Acc<E>& a, float& lse, float (&m)[E]) {
  lse = a.M + zlog(a.S);
  const float inv = __builtin_amdgcn_rcpf(a.S);
#pragma unroll
  for (int e = 0; e < E; ++e) m[e] = a.V[e] * inv;
}

// m~ = m rounded to bf16 (nearest even, v_cvt_pk_bf16_f32), packed in pairs, and its values.
template <int E> __device__ __forceinline__ void round_bf16(const float (&m)[E], uint32_t (&w)[E / 2], float (&mt)[E]) {
  typedef float f2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int i = 0; i < E / 2; ++i) {
    const b2_t p = __builtin_convertvector(f2_t{m[2 * i], m[2 * i + 1]}, b2_t);
    w[i] = __builtin_bit_cast(uint32_t, p);
    mt[2 * i] = __uint_as_float(w[i] << 16);
    mt[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
// Streaming (nontemporal) stores: a tree is written once and read by later routes, so its
// lines need not stay in the caches on the way out.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
template <int E> __device__ __forceinline__ void store_words(__bf16* p, const uint32_t (&w)[E / 2]) {
  if constexpr (E == 8) __builtin_nontemporal_store(u32x4_t{w[0], w[1], w[2], w[3]}, (u32x4_t*)p);
  else __builtin_nontemporal_store(u32x2_t{w[0], w[1]}, (u32x2_t*)p);
}
// This lane's part of r.m~ (the row's 16 lanes are summed by sum16).
template <int E> __device__ __forceinline__ float dot_part(const float (&rv)[E], const float (&mt)[E]) {
  float s = rv[0] * mt[0];
#pragma unroll
  for (int e = 1; e < E; ++e) s = __builtin_fmaf(rv[e], mt[e], s);
  return s;
}
template <int E, int D> __device__ __forceinline__ void ref_slice(const float* rfl, int r, int c, float (&rv)[E]) {
#pragma unroll
  for (int h = 0; h < E / 4; ++h) {
    const float4 q = *(const float4*)(rfl + r * D + E * c + 4 * h);
    rv[4 * h] = q.x; rv[4 * h + 1] = q.y; rv[4 * h + 2] = q.z; rv[4 * h + 3] = q.w;
  }
}

// Stores row r (< R) of node j of level l from lane c's slice: m~ and b = LSE - r.m~ (SF: the
// storage format, as in emit).
template <int E, int D, int SF>
__device__ __forceinline__ void emit_row(const BuildArgs& a, int u, int l, int64_t j, int r, int c, const float (&rv)[E],
                                         float lse, const float (&m)[E]) {
  if constexpr (SF != 0) {
    emit<__bf16, E, D, SF>(a, u, l, j, r, c, rv, lse, m);
    return;
  }
  const int64_t row = ((int64_t)u * a.cap[l] + j) * a.R + r;
  uint32_t w[E / 2];
  float mt[E];
  round_bf16<E>(m, w, mt);
  store_words<E>((__bf16*)a.m[l] + row * D + E * c, w);
  const float s = sum16(dot_part<E>(rv, mt));
  if (c == 0) __builtin_nontemporal_store(lse - s, a.b[l] + row);
}

// This lane's reference slices R[4 g + v][E c .. E c + E] in registers.
template <int E, int D> __device__ __forceinline__ void ref_slices4(const float* rfl, int g, int c, float (&rf)[4][E]) {
#pragma unroll
  for (int v = 0; v < 4; ++v) ref_slice<E, D>(rfl, 4 * g + v, c, rf[v]);
}

// Stores node j of level l from node layout (rows >= R skipped); the same values as emit_row
// row by row.  rf as in ref_slices4.
template <int E, int D, int SF>
__device__ __forceinline__ void emit4(const BuildArgs& a, int u, int l, int64_t j, int g, int c, const float (&rf)[4][E],
                                      const float (&lse)[4], const float (&m)[4][E]) {
  if constexpr (SF != 0) {
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (4 * g + v < a.R) emit<__bf16, E, D, SF>(a, u, l, j, 4 * g + v, c, rf[v], lse[v], m[v]);
    return;
  }
  const int64_t row0 = ((int64_t)u * a.cap[l] + j) * a.R + 4 * g;
  __bf16* mp = (__bf16*)a.m[l] + row0 * D + E * c;
  float dot[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    uint32_t w[E / 2];
    float mt[E];
    round_bf16<E>(m[v], w, mt);
    if (4 * g + v < a.R) store_words<E>(mp + v * D, w);
    dot[v] = dot_part<E>(rf[v], mt);
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) dot[v] = sum16(dot[v]);
  if (c < 4 && 4 * g + c < a.R) {
    const float bv = c == 0 ? lse[0] - dot[0] : c == 1 ? lse[1] - dot[1] : c == 2 ? lse[2] - dot[2] : lse[3] - dot[3];
    __builtin_nontemporal_store(bv, a.b[l] + row0 + c);
  }
}

// Accumulators of the four rows a lane holds, and their node-layout record [2 + E][64] float4:
// (M of rows 0..3), (S of rows 0..3), then V row by row, four elements per quad.
template <int E> struct Acc4 { Acc<E> a[4]; };

template <int E> __device__ __forceinline__ void acc4_clear(Acc4<E>& x) {
#pragma unroll
  for (int v = 0; v < 4; ++v) acc_clear(x.a[v]);
}
template <int E> __device__ __forceinline__ void acc4_fold(Acc4<E>& x, const float (&lse)[4], const float (&m)[4][E]) {
#pragma unroll
  for (int v = 0; v < 4; ++v) fold_row(x.a[v], lse[v], m[v]);
}
template <int E> __device__ __forceinline__ void acc4_finish(const Acc4<E>& x, float (&lse)[4], float (&m)[4][E]) {
#pragma unroll
  for (int v = 0; v < 4; ++v) finish_row(x.a[v], lse[v], m[v]);
}
template <int E> __device__ __forceinline__ void acc4_put(float4* p, int lane, const Acc4<E>& x) {
  p[lane] = make_float4(x.a[0].M, x.a[1].M, x.a[2].M, x.a[3].M);
  p[64 + lane] = make_float4(x.a[0].S, x.a[1].S, x.a[2].S, x.a[3].S);
#pragma unroll
  for (int v = 0; v < 4; ++v)
#pragma unroll
    for (int h = 0; h < E / 4; ++h)
      p[(2 + v * (E / 4) + h) * 64 + lane] =
          make_float4(x.a[v].V[4 * h], x.a[v].V[4 * h + 1], x.a[v].V[4 * h + 2], x.a[v].V[4 * h + 3]);
}
template <int E> __device__ __forceinline__ void acc4_get(const float4* p, int lane, Acc4<E>& x) {
  const float4 M = p[lane], S = p[64 + lane];
  x.a[0].M = M.x; x.a[1].M = M.y; x.a[2].M = M.z; x.a[3].M = M.w;
  x.a[0].S = S.x; x.a[1].S = S.y; x.a[2].S = S.z; x.a[3].S = S.w;
#pragma unroll
  for (int v = 0; v < 4; ++v)
#pragma unroll
    for (int h = 0; h < E / 4; ++h) {
      const float4 q = p[(2 + v * (E / 4) + h) * 64 + lane];
      x.a[v].V[4 * h] = q.x; x.a[v].V[4 * h + 1] = q.y; x.a[v].V[4 * h + 2] = q.z; x.a[v].V[4 * h + 3] = q.w;
    }
}
// Row v of a lane's record, for a thread that holds one row (the upper-level kernel).
template <int E> __device__ __forceinline__ void acc_put_row(float4* p, int lane, int v, const Acc<E>& x) {
  float* f = (float*)p;
  f[lane * 4 + v] = x.M;
  f[(64 + lane) * 4 + v] = x.S;
#pragma unroll
  for (int e = 0; e < E; ++e) f[((2 + v * (E / 4) + e / 4) * 64 + lane) * 4 + (e & 3)] = x.V[e];
}

// Spine record of level l of unit u: [U][L + 1][2 + E][64] float4 (levels 3..L used).
template <int E> __device__ __forceinline__ float4* spine4(const BuildArgs& a, int u, int l) {
  return (float4*)a.spine + ((int64_t)u * (a.L + 1) + l) * (2 + E) * 64;
}

// fp32 (LSE, mean) of level-4 node j for the upper levels, [U][cap_4][R] and [U][cap_4][R][D].
template <int E, int D>
__device__ __forceinline__ void put_sub4(const BuildArgs& a, int u, int64_t j, int g, int c, const float (&lse)[4],
                                         const float (&m)[4][E]) {
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int r = 4 * g + v;
    if (r >= a.R) continue;
    const int64_t row = ((int64_t)u * a.cap[a.S] + j) * a.R + r;
    float* mp = a.sub_m + row * D + E * c;
#pragma unroll
    for (int h = 0; h < E / 4; ++h)
      *(float4*)(mp + 4 * h) = make_float4(m[v][4 * h], m[v][4 * h + 1], m[v][4 * h + 2], m[v][4 * h + 3]);
    if (c == 0) a.sub_lse[row] = lse[v];
  }
}
template <int E, int D>
__device__ __forceinline__ void get_sub_row(const BuildArgs& a, int u, int64_t j, int r, int c, float& lse, float (&m)[E]) {
  if (r < a.R) {
    const int64_t row = ((int64_t)u * a.cap[a.S] + j) * a.R + r;
    const float* mp = a.sub_m + row * D + E * c;
#pragma unroll
    for (int h = 0; h < E / 4; ++h) {
      const float4 q = *(const float4*)(mp + 4 * h);
      m[4 * h] = q.x; m[4 * h + 1] = q.y; m[4 * h + 2] = q.z; m[4 * h + 3] = q.w;
    }
    lse = a.sub_lse[row];
  } else {
    lse = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) m[e] = 0.0f;
  }
}

// A finished level-3 node in LDS for the workgroup's level-4 fold: LSE [16], mean [16][D].
template <int E, int D>
__device__ __forceinline__ void put_slot(float* slot, int g, int c, const float (&lse)[4], const float (&m)[4][E]) {
  if (c == 0) *(float4*)(slot + 4 * g) = make_float4(lse[0], lse[1], lse[2], lse[3]);
#pragma unroll
  for (int v = 0; v < 4; ++v)
#pragma unroll
    for (int h = 0; h < E / 4; ++h)
      *(float4*)(slot + 16 + (4 * g + v) * D + E * c + 4 * h) =
          make_float4(m[v][4 * h], m[v][4 * h + 1], m[v][4 * h + 2], m[v][4 * h + 3]);
}
template <int E, int D>
__device__ __forceinline__ void get_slot(const float* slot, int g, int c, float (&lse)[4], float (&m)[4][E]) {
  const float4 l4 = *(const float4*)(slot + 4 * g);
  lse[0] = l4.x; lse[1] = l4.y; lse[2] = l4.z; lse[3] = l4.w;
#pragma unroll
  for (int v = 0; v < 4; ++v)
#pragma unroll
    for (int h = 0; h < E / 4; ++h) {
      const float4 q = *(const float4*)(slot + 16 + (4 * g + v) * D + E * c + 4 * h);
      m[v][4 * h] = q.x; m[v][4 * h + 1] = q.y; m[v][4 * h + 2] = q.z; m[v][4 * h + 3] = q.w;
    }
}

// Finished node j of level l0 into its ancestors up to ltop, node layout, accumulators of
// levels lbase.. in LDS ([level - lbase][2 + E][64]); as push_node.
template <int E, int D, int SF>
__device__ __forceinline__ void push4(const BuildArgs& a, float4* st, int lbase, int u, int l0, int j, int ltop, int g,
                                      int c, int lane, const float (&rf)[4][E], float (&lse)[4], float (&m)[4][E]) {
  int idx = j;
  for (int l = l0 + 1; l <= ltop; ++l) {
    float4* p = st + (l - lbase) * (2 + E) * 64;
    Acc4<E> acc;
    acc4_get(p, lane, acc);
    acc4_fold(acc, lse, m);
    if ((idx & 3) != 3) {
      acc4_put(p, lane, acc);
      return;
    }
    idx >>= 2;
    acc4_finish(acc, lse, m);
    emit4<E, D, SF>(a, u, l, idx, g, c, rf, lse, m);
    acc4_clear(acc);
    acc4_put(p, lane, acc);
  }
}

// Open nodes of levels l0..l1 for a unit with n1 leaves, node layout, accumulators in LDS; as
// flush_open.
template <int E, int D, int SF>
__device__ __forceinline__ void flush4(const BuildArgs& a, const float4* st, int lbase, int u, int64_t n1, int l0, int l1,
                                       int g, int c, int lane, const float (&rf)[4][E], bool& carry, float (&clse)[4],
                                       float (&cm)[4][E]) {
  for (int l = l0; l <= l1; ++l) {
    if (n1 % a.lpn[l] == 0) {
      carry = false;
      continue;
    }
    Acc4<E> acc;
    acc4_get(st + (l - lbase) * (2 + E) * 64, lane, acc);
    if (carry) acc4_fold(acc, clse, cm);
    acc4_finish(acc, clse, cm);
    emit4<E, D, SF>(a, u, l, (n1 - 1) / a.lpn[l], g, c, rf, clse, cm);
    carry = true;
  }
}

// One workgroup (four waves) per 64 leaves of a unit: levels 1..min(L, 4).
template <int D, int SF>
__global__ __launch_bounds__(256, 2) void zha_build_c4_kernel(BuildArgs a) {
  write_geo(a);
  constexpr int E = D / 16, RST = D + 8;
  extern __shared__ float lds[];
  __bf16* rsl = (__bf16*)lds;                  // [3][16][RST] reference parts
  float* rfl = lds + 24 * RST;                 // [16][D] references
  float* wsx = rfl + 16 * D;                   // [4][C4_WS] per-wave exchange
  float* hand = wsx + 4 * C4_WS;               // [4][c4_slot_floats(D)] per-wave slots
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int u = blockIdx.y, bi = u / a.Hkv, gh = u % a.Hkv;
  const int n1 = (int)(a.len.n[bi] / 4);
  const int L = a.L;
  const int j = blockIdx.x;
  const int c0 = j * 64;
  if (c0 >= n1) {
    if (j == 0 && w == 0) {  // no complete leaf: the unit's spine is empty
      Acc4<E> z;
      acc4_clear(z);
      for (int l = 3; l <= min(L, 4); ++l) acc4_put(spine4<E>(a, u, l), lane, z);
    }
    return;
  }
  refs_split<D>(a, gh, rsl, rfl, tid, 256);
  const int c1 = min(c0 + 64, n1);
  const int a0 = c0 + 16 * w, a1 = min(a0 + 16, c1);  // this wave's leaves
  float* ws = wsx + w * C4_WS;
  float* slot = hand + w * c4_slot_floats(D);
  float4* acc3p = (float4*)slot;  // the level-3 accumulator until the wave's node is finished
  if (L >= 3) {
    Acc4<E> z;
    acc4_clear(z);
    acc4_put(acc3p, lane, z);
  }
  __syncthreads();
  float rf[4][E];
  ref_slices4<E, D>(rfl, g, c, rf);
  if (a0 < a1) {
    const __bf16* Kb = (const __bf16*)a.K + ((int64_t)bi * a.Hkv + gh) * a.T * D;
    const int64_t tlast = 4 * (int64_t)n1 - 1;
    const int tau0 = a0 >> 2, tau1 = (a1 - 1) >> 2;
    Tile4<D> cur, nxt;
    load_tile4<D>(Kb, 16 * (int64_t)tau0, tlast, g, c, cur);
    for (int tau = tau0; tau <= tau1; ++tau) {
      if (tau < tau1) load_tile4<D>(Kb, 16 * (int64_t)(tau + 1), tlast, g, c, nxt);
      const int nl = min(4, a1 - 4 * tau);  // complete leaves in the tile
      tile_weights<D>(cur, rsl, g, c, nl, L >= 2, ws);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (q >= nl) break;
        float lse[4], m[4][E];
        leaf_mean4<D>(cur.kw[q], q, g, c, ws, lse, m);
        emit4<E, D, SF>(a, u, 1, 4 * tau + q, g, c, rf, lse, m);
      }
      if (L >= 2) {
        float lse[4], m[4][E];
        level2_mean4<D>(cur, g, c, ws, lse, m);
        emit4<E, D, SF>(a, u, 2, tau, g, c, rf, lse, m);  // complete, or the unit's open level-2 node
        if (L >= 3) {
          Acc4<E> acc3;
          acc4_get(acc3p, lane, acc3);
          if (nl == 4) {
            acc4_fold(acc3, lse, m);
            if ((tau & 3) == 3) {  // the wave's level-3 node is complete (its last tile)
              acc4_finish(acc3, lse, m);
              emit4<E, D, SF>(a, u, 3, tau >> 2, g, c, rf, lse, m);
              if (L >= 4) put_slot<E, D>(slot, g, c, lse, m);
              acc4_clear(acc3);
            } else {
              acc4_put(acc3p, lane, acc3);
            }
          }
          if (tau == tau1 && a1 == n1) {  // the unit's last tile: its open accumulator, open nodes
            acc4_put(spine4<E>(a, u, 3), lane, acc3);
            if (n1 % 16 != 0) {  // the open level-3 node, with the open level-2 node (nl < 4)
              if (nl < 4) acc4_fold(acc3, lse, m);
              acc4_finish(acc3, lse, m);
              emit4<E, D, SF>(a, u, 3, tau >> 2, g, c, rf, lse, m);
              if (L >= 4) put_slot<E, D>(slot, g, c, lse, m);
            }
          }
        }
      }
      wave_lds_sync();  // the next tile rewrites the exchange area
      cur = nxt;
    }
  }
  if (L < 4) return;
  __syncthreads();
  if (w != 0) return;
  Acc4<E> acc4;
  acc4_clear(acc4);
  const int nfull = (c1 - c0) >> 4;
  for (int sI = 0; sI < nfull; ++sI) {
    float lse[4], m[4][E];
    get_slot<E, D>(hand + sI * c4_slot_floats(D), g, c, lse, m);
    acc4_fold(acc4, lse, m);
  }
  if (c1 - c0 == 64) {
    float lse[4], m[4][E];
    acc4_finish(acc4, lse, m);
    acc4_clear(acc4);
    emit4<E, D, SF>(a, u, 4, j, g, c, rf, lse, m);
    if (L > 4) put_sub4<E, D>(a, u, j, g, c, lse, m);
  }
  if (c1 == n1) {
    acc4_put(spine4<E>(a, u, 4), lane, acc4);
    if (n1 % 64 != 0) {  // the open level-4 node: its complete children and the open level-3 node
      float lse[4], m[4][E];
      Acc4<E> t = acc4;
      if (n1 % 16 != 0) {
        get_slot<E, D>(hand + nfull * c4_slot_floats(D), g, c, lse, m);
        acc4_fold(t, lse, m);
      }
      acc4_finish(t, lse, m);
      emit4<E, D, SF>(a, u, 4, j, g, c, rf, lse, m);
      if (L > 4) put_sub4<E, D>(a, u, j, g, c, lse, m);
    }
  }
}

// One workgroup per (top node, unit): levels 5..L from the level-4 nodes.  Thread (w, g, c)
// holds reference row r = 4 g + w, elements E c .. E c + E -- row w of lane (g, c)'s node
// layout, so every value is computed as the node-layout kernels compute it.
template <int D, int SF>
__global__ __launch_bounds__(256) void zha_build_upper_c4_kernel(BuildArgs a) {
  constexpr int E = D / 16;
  extern __shared__ float ldsu[];  // accumulators of levels 5..L [L - 4][2 + E][256], references [16][D]
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int r = 4 * g + w;
  const int u = blockIdx.y, gh = u % a.Hkv;
  const int64_t n1 = a.len.n[u / a.Hkv] / 4;
  const int64_t nS_done = n1 / 64, nS_all = (n1 + 63) / 64;
  const int64_t cpt = a.lpn[a.L] / 64;  // level-4 nodes per top node
  const int64_t T0 = blockIdx.x, j0 = T0 * cpt;
  Stack<E> st{ldsu, 256, tid, 5};
  if (j0 >= nS_all) {
    if (T0 == 0) {
      Acc<E> z;
      acc_clear(z);
      for (int l = 5; l <= a.L; ++l) acc_put_row(spine4<E>(a, u, l), lane, w, z);
    }
    return;
  }
  float* rfl = ldsu + (a.L - 4) * (2 + E) * 256;
  for (int i = tid; i < 16 * D; i += 256) rfl[i] = i / D < a.R ? a.refs[((int64_t)gh * a.R) * D + i] : 0.0f;
  stack_clear(st, 5, a.L);
  __syncthreads();
  float rv[E];
  ref_slice<E, D>(rfl, r, c, rv);
  const int64_t j1 = min(j0 + cpt, nS_done);
  float lse = 0.0f, m[E];
  if (j0 < j1) get_sub_row<E, D>(a, u, j0, r, c, lse, m);
  for (int64_t jj = j0; jj < j1; ++jj) {
    float nlse = 0.0f, nm[E];
    if (jj + 1 < j1) get_sub_row<E, D>(a, u, jj + 1, r, c, nlse, nm);  // next child in flight
    int idx = (int)jj;
    for (int l = 5; l <= a.L; ++l) {
      Acc<E> acc;
      st.get(l, acc);
      fold_row(acc, lse, m);
      if ((idx & 3) != 3) {
        st.put(l, acc);
        break;
      }
      idx >>= 2;
      finish_row(acc, lse, m);
      if (r < a.R) emit_row<E, D, SF>(a, u, l, idx, r, c, rv, lse, m);
      acc_clear(acc);
      st.put(l, acc);
    }
    lse = nlse;
#pragma unroll
    for (int e = 0; e < E; ++e) m[e] = nm[e];
  }
  if (j0 + cpt >= nS_all) {  // the unit's last top node
    for (int l = 5; l <= a.L; ++l) {
      Acc<E> x;
      st.get(l, x);
      acc_put_row(spine4<E>(a, u, l), lane, w, x);
    }
    bool carry = n1 % 64 != 0;  // the open level-4 node, written by the workgroup kernel
    float clse = 0.0f, cm[E];
#pragma unroll
    for (int e = 0; e < E; ++e) cm[e] = 0.0f;
    if (carry) get_sub_row<E, D>(a, u, nS_all - 1, r, c, clse, cm);
    for (int l = 5; l <= a.L; ++l) {
      if (n1 % a.lpn[l] == 0) {
        carry = false;
        continue;
      }
      Acc<E> acc;
      st.get(l, acc);
      if (carry) fold_row(acc, clse, cm);
      finish_row(acc, clse, cm);
      if (r < a.R) emit_row<E, D, SF>(a, u, l, (n1 - 1) / a.lpn[l], r, c, rv, clse, cm);
      carry = true;
    }
  }
}

// One wave per unit: the leaves completed by the new rows, through every level.
template <int D, int SF>
__global__ __launch_bounds__(64) void zha_append_c4_kernel(BuildArgs a) {
  write_geo(a);
  constexpr int E = D / 16, RST = D + 8;
  extern __shared__ float lds[];
  __bf16* rsl = (__bf16*)lds;                  // [3][16][RST]
  float* rfl = lds + 24 * RST;                 // [16][D]
  float* ws = rfl + 16 * D;                    // [C4_WS]
  float4* st4 = (float4*)(ws + C4_WS);         // levels 3..L: [L - 2][2 + E][64]
  const int lane = threadIdx.x, g = lane >> 4, c = lane & 15;
  const int u = blockIdx.x, bi = u / a.Hkv, gh = u % a.Hkv;
  const int64_t n1_old = a.len_prev.n[bi] / 4, n1 = a.len.n[bi] / 4;
  if (n1 == n1_old) return;
  refs_split<D>(a, gh, rsl, rfl, lane, 64);
  for (int l = 3; l <= a.L; ++l) {
    Acc4<E> x;
    acc4_get(spine4<E>(a, u, l), lane, x);
    acc4_put(st4 + (l - 3) * (2 + E) * 64, lane, x);
  }
  __syncthreads();
  float rf[4][E];
  ref_slices4<E, D>(rfl, g, c, rf);
  const __bf16* Kb = (const __bf16*)a.K + ((int64_t)bi * a.Hkv + gh) * a.T * D;
  const int64_t tlast = 4 * n1 - 1;
  for (int64_t leaf = n1_old; leaf < n1; ++leaf) {
    const int q = (int)(leaf & 3);
    const bool done2 = a.L >= 2 && q == 3;  // the leaf completes its level-2 node
    Tile4<D> tk;
    load_tile4<D>(Kb, 16 * (leaf >> 2), tlast, g, c, tk);
    tile_weights<D>(tk, rsl, g, c, 4, done2, ws);
    float lse[4], m[4][E];
    const typename KwVec<E>::type kwq = q == 0 ? tk.kw[0] : q == 1 ? tk.kw[1] : q == 2 ? tk.kw[2] : tk.kw[3];
    leaf_mean4<D>(kwq, q, g, c, ws, lse, m);
    emit4<E, D, SF>(a, u, 1, leaf, g, c, rf, lse, m);
    if (done2) {
      level2_mean4<D>(tk, g, c, ws, lse, m);
      emit4<E, D, SF>(a, u, 2, leaf >> 2, g, c, rf, lse, m);
      push4<E, D, SF>(a, st4, 3, u, 2, (int)(leaf >> 2), a.L, g, c, lane, rf, lse, m);
    }
    wave_lds_sync();
  }
  for (int l = 3; l <= a.L; ++l) {
    Acc4<E> x;
    acc4_get(st4 + (l - 3) * (2 + E) * 64, lane, x);
    acc4_put(spine4<E>(a, u, l), lane, x);
  }
  bool carry = false;
  float clse[4], cm[4][E];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    clse[v] = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) cm[v][e] = 0.0f;
  }
  if (a.L >= 2 && n1 % 4 != 0) {  // the open level-2 node, from its complete leaves' tokens
    const int64_t tau = (n1 - 1) >> 2;
    Tile4<D> tk;
    load_tile4<D>(Kb, 16 * tau, tlast, g, c, tk);
    tile_weights<D>(tk, rsl, g, c, (int)(n1 & 3), true, ws);
    level2_mean4<D>(tk, g, c, ws, clse, cm);
    emit4<E, D, SF>(a, u, 2, tau, g, c, rf, clse, cm);
    carry = true;
  }
  flush4<E, D, SF>(a, st4, 3, u, n1, 3, a.L, g, c, lane, rf, carry, clse, cm);
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

// One node-layout accumulator record of the matrix-core path: [2 + d/16][64] float4.
size_t c4_record_bytes(int d) { return (size_t)(2 + d / 16) * 64 * 4 * sizeof(float); }
size_t c4_build_lds(int d) {
  return (size_t)(3 * 16 * (d + 8)) * 2 + (16 * (size_t)d + 4 * C4_WS + 4 * (size_t)c4_slot_floats(d)) * sizeof(float);
}
size_t c4_upper_lds(int L, int d) {
  return ((size_t)(L > 4 ? L - 4 : 0) * (2 + d / 16) * 256 + 16 * (size_t)d) * sizeof(float);
}
size_t c4_append_lds(int L, int d) {
  return (size_t)(3 * 16 * (d + 8)) * 2 + (16 * (size_t)d + C4_WS) * sizeof(float) +
         (size_t)(L > 2 ? L - 2 : 0) * c4_record_bytes(d);
}

}  // namespace

// LDS accumulator stack of nlev levels; the spine in HBM keeps levels 0..L (0 and 1 unused).
size_t zha_stack_bytes(int nlev, int d, int R) {
  return (size_t)(nlev > 0 ? nlev : 0) * (d / 16 + 2) * (16 * R) * sizeof(float);
}

// The spine holds levels 0..L in whichever layout the tree's build path uses (the larger).
size_t zha_spine_bytes(int L, int d, int R) {
  const size_t a = zha_stack_bytes(L + 1, d, R), b = (size_t)(L + 1) * c4_record_bytes(d);
  return a > b ? a : b;
}

bool zha_build_c4_path(int C, int esize) { return C == 4 && esize == 2; }

// Largest dynamic LDS any build kernel of the tree's path asks for.
size_t zha_build_lds_bytes(int C, int S, int L, int d, int R, int esize) {
  if (zha_build_c4_path(C, esize)) {
    size_t m = c4_build_lds(d);
    if (c4_upper_lds(L, d) > m) m = c4_upper_lds(L, d);
    if (c4_append_lds(L, d) > m) m = c4_append_lds(L, d);
    return m;
  }
  size_t m = zha_stack_bytes(S - 1, d, R);                         // subtree
  if (zha_stack_bytes(L - S, d, R) > m) m = zha_stack_bytes(L - S, d, R);  // upper
  if (zha_stack_bytes(L - 1, d, R) > m) m = zha_stack_bytes(L - 1, d, R);  // append
  return m;
}

namespace {

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

template <int D, int SF>
hipError_t launch_build_c4(zha_tree* t, const BuildArgs& a, hipStream_t s) {
  const size_t sh = c4_build_lds(D);
  hipError_t e = allow_lds(zha_build_c4_kernel<D, SF>, sh);
  if (e != hipSuccess) return e;
  const int64_t groups = (t->cap[1] + 63) / 64;
  zha_time_begin(t, s, ZHA_K_BUILD, t->S);
  hipLaunchKernelGGL((zha_build_c4_kernel<D, SF>), dim3((unsigned)(groups > 0 ? groups : 1), (unsigned)t->U), dim3(256),
                     sh, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  zha_time_end(t, s, ZHA_K_BUILD, t->S);
  if (t->L <= 4) return hipSuccess;
  const size_t sh_up = c4_upper_lds(t->L, D);
  e = allow_lds(zha_build_upper_c4_kernel<D, SF>, sh_up);
  if (e != hipSuccess) return e;
  zha_time_begin(t, s, ZHA_K_BUILD, t->L);
  hipLaunchKernelGGL((zha_build_upper_c4_kernel<D, SF>),
                     dim3((unsigned)(t->cap[t->L] > 0 ? t->cap[t->L] : 1), (unsigned)t->U), dim3(256), sh_up, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  zha_time_end(t, s, ZHA_K_BUILD, t->L);
  return hipSuccess;
}

template <int D, int SF>
hipError_t launch_append_c4(zha_tree* t, const BuildArgs& a, hipStream_t s) {
  const size_t sh = c4_append_lds(t->L, D);
  hipError_t e = allow_lds(zha_append_c4_kernel<D, SF>, sh);
  if (e != hipSuccess) return e;
  zha_time_begin(t, s, ZHA_K_APPEND, 0);
  hipLaunchKernelGGL((zha_append_c4_kernel<D, SF>), dim3((unsigned)t->U), dim3(64), sh, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  zha_time_end(t, s, ZHA_K_APPEND, 0);
  return hipSuccess;
}

// The matrix-core kernels for the tree's head dimension and summary format.
template <int D>
hipError_t launch_c4(zha_tree* t, const BuildArgs& a, hipStream_t s, bool append) {
  if (t->f4) return append ? launch_append_c4<D, 2>(t, a, s) : launch_build_c4<D, 2>(t, a, s);
  if (t->f8) return append ? launch_append_c4<D, 1>(t, a, s) : launch_build_c4<D, 1>(t, a, s);
  return append ? launch_append_c4<D, 0>(t, a, s) : launch_build_c4<D, 0>(t, a, s);
}

}  // namespace

// The subtree kernel is timed as build level S, the upper kernel as build level L.  Trees of
// bf16 keys with C = 4 take the matrix-core kernels, every other tree the per-thread ones;
// build and append of one tree always take the same path.
hipError_t zha_launch_build(zha_tree* t, const void* K, hipStream_t s) {
  BuildArgs a = make_args(t, K);
  if (zha_build_c4_path(t->C, t->desc.dtype == ZHA_BF16 ? 2 : 4))
    return t->d == 64 ? launch_c4<64>(t, a, s, false) : launch_c4<128>(t, a, s, false);
  if (t->desc.dtype == ZHA_BF16)
    return t->d == 64 ? launch_build_td<__bf16, 64>(t, a, s) : launch_build_td<__bf16, 128>(t, a, s);
  return t->d == 64 ? launch_build_td<float, 64>(t, a, s) : launch_build_td<float, 128>(t, a, s);
}

hipError_t zha_launch_append(zha_tree* t, const void* K, hipStream_t s) {
  BuildArgs a = make_args(t, K);
  if (zha_build_c4_path(t->C, t->desc.dtype == ZHA_BF16 ? 2 : 4))
    return t->d == 64 ? launch_c4<64>(t, a, s, true) : launch_c4<128>(t, a, s, true);
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
