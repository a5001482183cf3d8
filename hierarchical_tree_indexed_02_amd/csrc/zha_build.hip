// zha_build.hip -- summary tree construction and incremental growth.
//
// Every node stores, per reference query r, the tangent plane of its log
// attention mass at q = r ([wqu] "Building the tree"; page key in include/zha.h):
//   LSE_r = log sum_{t in node} exp(r.k_t),  m_r = sum_t softmax_t(r.k) k_t,
//   b_r = LSE_r - r.m~_r  with m~_r the stored (rounded) m_r,
// so the plane b_r + q.m~_r is exact at q = r for the stored values.  Leaves
// cover C raw tokens; a parent is the exact log-sum-exp combination of its C
// children's fp32 (LSE, mean) ([aitop] abstract: recursively compressed key
// summaries).  One workgroup streams one top node's tokens in order: tokens
// fold into the leaf accumulator (registers), each finished leaf folds into
// its parent's accumulator (LDS), and each finished node cascades upward.
// Thread (r, lane) owns reference query r and a 16th of the head dimension.
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
  int64_t cap[ZHA_MAX_LEVELS + 2];
  int64_t lpn[ZHA_MAX_LEVELS + 2];  // leaves per node at level l: C^(l-1)
  float* spine;             // [U][L+1][E+2][NT]
  int L, C, R, Hkv;
  int64_t T;
  ZLens len;                // lengths after the operation
  ZLens len_prev;           // append: lengths before it
};

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

// (LSE, mean slice) of leaf chunk c of this unit from its C raw keys.
template <typename T, int E, int D>
__device__ __forceinline__ void leaf_planes(const T* Kb, int64_t c, int C, int ln, const float (&rv)[E], float& lse,
                                            float (&m)[E]) {
  Acc<E> acc;
  acc_clear(acc);
  for (int t = 0; t < C; ++t) {
    float k[E];
    load_slice<T, E>(Kb + (c * C + t) * D + ln * E, k);
    const float x = dot_slice<E>(rv, k);
    acc_fold(acc, x, k);
  }
  acc_finish(acc, lse, m);
}

// Store node j of level l: m~ = m rounded to the storage type, b = LSE - r.m~.
template <typename T, int E, int D>
__device__ __forceinline__ void emit(const BuildArgs& a, int u, int l, int64_t j, int r, int ln, const float (&rv)[E],
                                     float lse, const float (&m)[E]) {
  T* mp = (T*)a.m[l] + (((int64_t)u * a.cap[l] + j) * a.R + r) * D + ln * E;
  float mt[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const T x = Mf<T>::from_f32(m[e]);
    mp[e] = x;
    mt[e] = Mf<T>::to_f32(x);
  }
  const float rm = dot_slice<E>(rv, mt);
  if (ln == 0) a.b[l][((int64_t)u * a.cap[l] + j) * a.R + r] = lse - rm;
}

// Accumulator stack of levels 2..L in LDS, struct-of-arrays [l][E+2][NT].
template <int E> struct Stack {
  float* base;
  int NT, tid;
  __device__ float& M(int l) { return base[((int64_t)l * (E + 2) + 0) * NT + tid]; }
  __device__ float& S(int l) { return base[((int64_t)l * (E + 2) + 1) * NT + tid]; }
  __device__ float& V(int l, int e) { return base[((int64_t)l * (E + 2) + 2 + e) * NT + tid]; }
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

// Leaf c is finished: store it, fold it into its ancestors, finishing every
// ancestor whose last child it is.
template <typename T, int E, int D>
__device__ __forceinline__ void push_leaf(const BuildArgs& a, Stack<E>& st, int u, int64_t c, int r, int ln,
                                          const float (&rv)[E], float lse, float (&m)[E]) {
  emit<T, E, D>(a, u, 1, c, r, ln, rv, lse, m);
  for (int l = 2; l <= a.L; ++l) {
    Acc<E> acc;
    st.get(l, acc);
    acc_fold(acc, lse, m);
    if ((c + 1) % a.lpn[l] != 0) {
      st.put(l, acc);
      return;
    }
    acc_finish(acc, lse, m);
    emit<T, E, D>(a, u, l, c / a.lpn[l], r, ln, rv, lse, m);
    acc_clear(acc);
    st.put(l, acc);
  }
}

// Writes the open (partial) node of every level for a unit with n1 leaves.
template <typename T, int E, int D>
__device__ __forceinline__ void flush_open(const BuildArgs& a, Stack<E>& st, int u, int64_t n1, int r, int ln,
                                           const float (&rv)[E]) {
  bool carry = false;
  float clse = 0.0f, cm[E];
#pragma unroll
  for (int e = 0; e < E; ++e) cm[e] = 0.0f;
  for (int l = 2; l <= a.L; ++l) {
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
__device__ __forceinline__ void stack_clear(Stack<E>& st, int L) {
  for (int l = 2; l <= L; ++l) {
    Acc<E> z;
    acc_clear(z);
    st.put(l, z);
  }
}

template <int E>
__device__ __forceinline__ void spine_io(const BuildArgs& a, Stack<E>& st, int u, bool store) {
  float* sp = a.spine + (int64_t)u * (a.L + 1) * (E + 2) * st.NT;
  for (int l = 2; l <= a.L; ++l)
    for (int f = 0; f < E + 2; ++f) {
      float* g = sp + ((int64_t)l * (E + 2) + f) * st.NT + st.tid;
      float* s = st.base + ((int64_t)l * (E + 2) + f) * st.NT + st.tid;
      if (store) *g = *s; else *s = *g;
    }
}

// One workgroup per (top node, unit); blockDim = 16 R.
template <typename T, int D>
__global__ __launch_bounds__(256) void zha_build_kernel(BuildArgs a) {
  constexpr int E = D / 16;
  extern __shared__ float lds_stack[];
  const int tid = threadIdx.x, r = tid >> 4, ln = tid & 15;
  const int u = blockIdx.y, bi = u / a.Hkv, g = u % a.Hkv;
  const int64_t N = a.len.n[bi];
  const int64_t n1 = N / a.C;
  const int64_t per_top = a.lpn[a.L];
  const int64_t j = blockIdx.x;
  const int64_t c0 = j * per_top;
  Stack<E> st{lds_stack, (int)blockDim.x, tid};
  if (c0 >= n1) {
    if (j == 0) {  // no complete leaf: the unit has an empty spine
      stack_clear(st, a.L);
      spine_io(a, st, u, true);
    }
    return;
  }
  const int64_t c1 = min(c0 + per_top, n1);
  float rv[E];
  load_slice<float, E>(a.refs + ((int64_t)g * a.R + r) * D + ln * E, rv);
  const T* Kb = (const T*)a.K + ((int64_t)bi * a.Hkv + g) * a.T * D;
  stack_clear(st, a.L);
  for (int64_t c = c0; c < c1; ++c) {
    float lse, m[E];
    leaf_planes<T, E, D>(Kb, c, a.C, ln, rv, lse, m);
    push_leaf<T, E, D>(a, st, u, c, r, ln, rv, lse, m);
  }
  if (c1 == n1) {  // rightmost top node: keep the open accumulators, write the open nodes
    spine_io(a, st, u, true);
    flush_open<T, E, D>(a, st, u, n1, r, ln, rv);
  }
}

// One workgroup per unit: fold the leaves completed by the new rows.
template <typename T, int D>
__global__ __launch_bounds__(256) void zha_append_kernel(BuildArgs a) {
  constexpr int E = D / 16;
  extern __shared__ float lds_stack[];
  const int tid = threadIdx.x, r = tid >> 4, ln = tid & 15;
  const int u = blockIdx.x, bi = u / a.Hkv, g = u % a.Hkv;
  const int64_t n1_old = a.len_prev.n[bi] / a.C;
  const int64_t n1 = a.len.n[bi] / a.C;
  if (n1 == n1_old) return;
  Stack<E> st{lds_stack, (int)blockDim.x, tid};
  float rv[E];
  load_slice<float, E>(a.refs + ((int64_t)g * a.R + r) * D + ln * E, rv);
  const T* Kb = (const T*)a.K + ((int64_t)bi * a.Hkv + g) * a.T * D;
  spine_io(a, st, u, false);
  for (int64_t c = n1_old; c < n1; ++c) {
    float lse, m[E];
    leaf_planes<T, E, D>(Kb, c, a.C, ln, rv, lse, m);
    push_leaf<T, E, D>(a, st, u, c, r, ln, rv, lse, m);
  }
  spine_io(a, st, u, true);
  flush_open<T, E, D>(a, st, u, n1, r, ln, rv);
}

#pragma clang fp contract(on)

BuildArgs make_args(const zha_tree* t, const void* K) {
  BuildArgs a;
  a.K = K;
  a.refs = t->refs;
  for (int l = 0; l < ZHA_MAX_LEVELS + 2; ++l) {
    a.m[l] = t->m[l];
    a.b[l] = t->b[l];
    a.cap[l] = t->cap[l];
    a.lpn[l] = l >= 1 ? t->span[l] / t->C : 1;
  }
  a.spine = t->spine;
  a.L = t->L;
  a.C = t->C;
  a.R = t->R;
  a.Hkv = t->desc.n_kv_heads;
  a.T = t->T;
  a.len = t->len;
  a.len_prev = t->len_prev;
  return a;
}

}  // namespace

size_t zha_stack_bytes(int L, int d, int R) {
  return (size_t)(L + 1) * (d / 16 + 2) * (16 * R) * sizeof(float);
}

// Kernels whose accumulator stack exceeds the default dynamic LDS limit opt in to more.
template <typename F>
hipError_t allow_lds(F kernel, size_t bytes) {
  return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

hipError_t zha_launch_build(zha_tree* t, const void* K, hipStream_t s) {
  BuildArgs a = make_args(t, K);
  const size_t sh = zha_stack_bytes(t->L, t->d, t->R);
  hipError_t e0 = t->desc.dtype == ZHA_BF16
                      ? (t->d == 64 ? allow_lds(zha_build_kernel<__bf16, 64>, sh) : allow_lds(zha_build_kernel<__bf16, 128>, sh))
                      : (t->d == 64 ? allow_lds(zha_build_kernel<float, 64>, sh) : allow_lds(zha_build_kernel<float, 128>, sh));
  if (e0 != hipSuccess) return e0;
  dim3 grid((unsigned)(t->cap[t->L] > 0 ? t->cap[t->L] : 1), (unsigned)t->U), block(16 * t->R);
  zha_time_begin(t, s, ZHA_K_BUILD, 0);
  if (t->desc.dtype == ZHA_BF16) {
    if (t->d == 64) hipLaunchKernelGGL((zha_build_kernel<__bf16, 64>), grid, block, sh, s, a);
    else hipLaunchKernelGGL((zha_build_kernel<__bf16, 128>), grid, block, sh, s, a);
  } else {
    if (t->d == 64) hipLaunchKernelGGL((zha_build_kernel<float, 64>), grid, block, sh, s, a);
    else hipLaunchKernelGGL((zha_build_kernel<float, 128>), grid, block, sh, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  zha_time_end(t, s, ZHA_K_BUILD, 0);
  return hipSuccess;
}

hipError_t zha_launch_append(zha_tree* t, const void* K, hipStream_t s) {
  BuildArgs a = make_args(t, K);
  const size_t sh = zha_stack_bytes(t->L, t->d, t->R);
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
