// zha_internal.h -- device helpers and host-side tree object of the ZHA library.
// Page references: see include/zha.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <vector>

#include "zha.h"

// ----------------------------------------------------------------------------- device types

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16;
typedef unsigned long long u64;

#define ZHA_LOG2E 1.4426950408889634f
#define ZHA_LN2 0.6931471805599453f

// exp and log on the hardware transcendental units (v_exp_f32 / v_log_f32 are base 2).
__device__ __forceinline__ float zexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float zexp(float x) { return __builtin_amdgcn_exp2f(x * ZHA_LOG2E); }
__device__ __forceinline__ float zlog(float x) { return __builtin_amdgcn_logf(x) * ZHA_LN2; }
__device__ __forceinline__ float zlog2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float bf16_bits_to_f32(u16 h) { return __uint_as_float((uint32_t)h << 16); }
// fp32 -> bf16, round to nearest even (finite values).
__device__ __forceinline__ u16 f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (u16)(u >> 16);
}

// Storage-type traits: how many elements one lane feeds a 16x16 MFMA per k-step.
//   bf16: v_mfma_f32_16x16x32_bf16, 8 elements per lane, k = 32 per instruction.
//   f32:  v_mfma_f32_16x16x4f32,   1 element per lane,  k = 4 per instruction.
// Lane i of the wave holds operand row/column (i % 16) and k-slot group (i / 16).
template <typename T> struct Mf;
template <> struct Mf<__bf16> {
  typedef bf16x8_t frag;
  static constexpr int EPL = 8;
  static constexpr int KPER = 32;
  __device__ static __forceinline__ frag load(const __bf16* p) { return *(const bf16x8_t*)p; }
  __device__ static __forceinline__ frag load_stream(const __bf16* p) { return __builtin_nontemporal_load((const bf16x8_t*)p); }
  __device__ static __forceinline__ frag zero() { bf16x8_t z; for (int e = 0; e < 8; ++e) z[e] = (__bf16)0.0f; return z; }
  __device__ static __forceinline__ f32x4_t mma(frag a, frag b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ float to_f32(__bf16 x) { return (float)x; }
  __device__ static __forceinline__ __bf16 from_f32(float x) {
    return __builtin_bit_cast(__bf16, f32_to_bf16_bits(x));
  }
};
template <> struct Mf<float> {
  typedef float frag;
  static constexpr int EPL = 1;
  static constexpr int KPER = 4;
  __device__ static __forceinline__ frag load(const float* p) { return *p; }
  __device__ static __forceinline__ frag load_stream(const float* p) { return __builtin_nontemporal_load(p); }
  __device__ static __forceinline__ frag zero() { return 0.0f; }
  __device__ static __forceinline__ f32x4_t mma(frag a, frag b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ float to_f32(float x) { return x; }
  __device__ static __forceinline__ float from_f32(float x) { return x; }
};

// ---------------------------------------------------------------- fp8 (OCP e4m3) summaries
//
// A row of m is stored as e4m3 codes times a power-of-two scale 2^e, e the smallest
// integer with max|m| * 2^-e <= 448 (the largest e4m3 value).  Encoding rounds m * 2^-e to
// the nearest e4m3 value, ties to even mantissa, subnormals (multiples of 2^-9 below 2^-6)
// kept; the hardware conversion does exactly this for inputs within +-448 (checked against
// enumeration of the format on every grid point, midpoint and near-midpoint; it keeps the
// sign of a negative value that rounds to zero, which decodes to the same zero).  Decoding
// uses the hardware conversion too (exact: every e4m3 value is a float).

// Scale exponent of a row whose largest magnitude is amax (0 for an all-zero row).
__device__ __forceinline__ int fp8_row_exp(float amax) {
  if (!(amax >= 1e-30f)) return 0;  // an all-zero (or negligible) row: every code is 0
  const uint32_t u = __float_as_uint(amax);
  const int ea = (int)((u >> 23) & 0xFF) - 127;   // amax = M * 2^ea, M in [1, 2) (normal amax)
  const uint32_t mant = u & 0x7FFFFFu;            // M > 1.75 <=> mantissa field > 0.75 * 2^23
  return ea - 8 + (mant > 0x600000u ? 1 : 0);
}

// fp4 (OCP e2m1) summaries: a row of m is cut into blocks of 32 values, each stored as e2m1
// codes (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), two per byte with element 2i in the low
// nibble of byte i, times a power-of-two scale 2^e, e the smallest integer with
// max|m_block| * 2^-e <= 6, kept as the byte e + 127.  The hardware conversion rounds to the
// nearest e2m1 value, ties to even mantissa (checked against enumeration of the format on
// grid points, midpoints and near-midpoints; a negative value that rounds to zero keeps its
// sign, which decodes to the same zero); decoding with the scale folded in is exact.

// Scale exponent of a block whose largest magnitude is amax (0 for an all-zero block).
__device__ __forceinline__ int fp4_block_exp(float amax) {
  if (!(amax >= 1e-30f)) return 0;
  const uint32_t u = __float_as_uint(amax);
  const int ea = (int)((u >> 23) & 0xFF) - 127;   // amax = M * 2^ea, M in [1, 2)
  const uint32_t mant = u & 0x7FFFFFu;            // M > 1.5 <=> mantissa field > 0.5 * 2^23
  return ea - 2 + (mant > 0x400000u ? 1 : 0);
}
// Scale 2^e of a stored scale byte e + 127.
__device__ __forceinline__ float fp4_scale(uint32_t byte) { return __uint_as_float(byte << 23); }

// Value of e4m3 code c (normal or subnormal; codes here never hold NaN).
__device__ __forceinline__ float fp8_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float v = e == 0u ? (float)m * 0.001953125f : __builtin_ldexpf(1.0f + (float)m * 0.125f, (int)e - 7);
  return (c & 0x80u) ? -v : v;
}

// Sum over each row of 16 lanes, the total left in every lane of the row, with four
// DPP adds (data-parallel-primitive lane moves within a row, no LDS round trip): swap
// neighbours, swap pairs (each lane then holds its quad's sum), add the half-row mirror
// (lanes i and 7-i: each lane holds its 8-lane half's sum), add the row mirror (lanes i
// and 15-i).  Fixed order: every caller gets the same bits for the same inputs.  Every
// source lane of these four patterns lies in the row, so bound_ctrl (zero for a lane with
// no source) never applies; it lets the compiler fold each move into the add or max that
// uses it (v_add_f32_dpp).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float sum16(float x) {
  x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);  // row_half_mirror
  x += dpp_mov<0x140>(x);  // row_mirror
  return x;
}
// Maximum over the 16 lanes of a DPP row, in every lane of the row (same moves as sum16).
__device__ __forceinline__ float max16(float x) {
  x = fmaxf(x, dpp_mov<0xB1>(x));
  x = fmaxf(x, dpp_mov<0x4E>(x));
  x = fmaxf(x, dpp_mov<0x141>(x));
  x = fmaxf(x, dpp_mov<0x140>(x));
  return x;
}

// Wave-wide reductions on gfx950 with every lane ending with the same bits: the row of 16
// lanes by DPP (as above), then the row pairs by v_permlane16_swap and the halves by
// v_permlane32_swap (each lane adds the same two values in the same order).
__device__ __forceinline__ float wave_sum(float x) {
  x = sum16(x);
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float wave_max(float x) {
  x = max16(x);
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  x = min(x, dpp_u32<0xB1>(x));
  x = min(x, dpp_u32<0x4E>(x));
  x = min(x, dpp_u32<0x141>(x));
  x = min(x, dpp_u32<0x140>(x));
  auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = min(a[0], a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return min(b[0], b[1]);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, dpp_u32<0xB1>(x));
  x = max(x, dpp_u32<0x4E>(x));
  x = max(x, dpp_u32<0x141>(x));
  x = max(x, dpp_u32<0x140>(x));
  auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = max(a[0], a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return max(b[0], b[1]);
}
__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long x) {
  auto step = [](unsigned long long v, uint32_t lo, uint32_t hi) { return v + (((unsigned long long)hi << 32) | lo); };
  x = step(x, dpp_u32<0xB1>((uint32_t)x), dpp_u32<0xB1>((uint32_t)(x >> 32)));
  x = step(x, dpp_u32<0x4E>((uint32_t)x), dpp_u32<0x4E>((uint32_t)(x >> 32)));
  x = step(x, dpp_u32<0x141>((uint32_t)x), dpp_u32<0x141>((uint32_t)(x >> 32)));
  x = step(x, dpp_u32<0x140>((uint32_t)x), dpp_u32<0x140>((uint32_t)(x >> 32)));
  auto al = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
  auto ah = __builtin_amdgcn_permlane16_swap((uint32_t)(x >> 32), (uint32_t)(x >> 32), false, false);
  x = ((((unsigned long long)ah[0]) << 32) | al[0]) + ((((unsigned long long)ah[1]) << 32) | al[1]);
  auto bl = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
  auto bh = __builtin_amdgcn_permlane32_swap((uint32_t)(x >> 32), (uint32_t)(x >> 32), false, false);
  return ((((unsigned long long)bh[0]) << 32) | bl[0]) + ((((unsigned long long)bh[1]) << 32) | bl[1]);
}

// fp32 accumulator of one (node, reference query) while its children are folded in:
// running maximum M, S = sum exp(x - M), V = sum exp(x - M) * m (this lane's slice).
// Folding child (x, m) and finishing give LSE = M + log S, mean = V / S, the exact
// log-sum-exp combination of the children ([aitop] abstract: recursive compression).
template <int E> struct Acc {
  float M, S;
  float V[E];
};

template <int E> __device__ __forceinline__ void acc_clear(Acc<E>& a) {
  a.M = -INFINITY;
  a.S = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) a.V[e] = 0.0f;
}

#pragma clang fp contract(off)
template <int E> __device__ __forceinline__ void acc_fold(Acc<E>& a, float x, const float (&m)[E]) {
  if (a.S == 0.0f) {
    a.M = x;
    a.S = 1.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) a.V[e] = m[e];
  } else if (x <= a.M) {
    float c = zexp(x - a.M);
    a.S = a.S + c;
#pragma unroll
    for (int e = 0; e < E; ++e) a.V[e] = __builtin_fmaf(c, m[e], a.V[e]);
  } else {
    float c = zexp(a.M - x);
    a.S = __builtin_fmaf(a.S, c, 1.0f);
#pragma unroll
    for (int e = 0; e < E; ++e) a.V[e] = __builtin_fmaf(a.V[e], c, m[e]);
    a.M = x;
  }
}

template <int E> __device__ __forceinline__ void acc_finish(const Acc<E>& a, float& lse, float (&m)[E]) {
  lse = a.M + zlog(a.S);
  const float inv = 1.0f / a.S;
#pragma unroll
  for (int e = 0; e < E; ++e) m[e] = a.V[e] * inv;
}
#pragma clang fp contract(on)

// Routing units are numbered ((sequence * Tq + query) * Hkv + KV head) * hr + head group:
// Tq queries per sequence, hr routing units per (query, KV head).  A unit's query heads are
// rows u * G' .. u * G' + G' - 1 of q [B][Tq][Hq][d] (G' = Gq / hr heads per unit); its
// planes and K/V are those of its (sequence, KV head) pair, returned here.
__device__ __forceinline__ int plane_unit(int u, int hr, int Hkv, int Tq) {
  const int x = u / hr;
  return (x / (Hkv * Tq)) * Hkv + x % Hkv;
}
// The unit's query index within its sequence's block of Tq queries.
__device__ __forceinline__ int unit_query(int u, int hr, int Hkv, int Tq) { return (u / hr / Hkv) % Tq; }
// The unit's union group, numbered (sequence, KV head, query chunk of TS queries; NTC chunks).
__device__ __forceinline__ int union_group(int u, int hr, int Hkv, int Tq, int TS, int NTC) {
  return plane_unit(u, hr, Hkv, Tq) * NTC + unit_query(u, hr, Hkv, Tq) / TS;
}

// ----------------------------------------------------------------------------- host side

#define ZHA_MAX_LEVELS 16
#define ZHA_MAX_TIMING 256
#define ZHA_MAX_BATCH 64

// Sequence lengths by value: the build, append and dense-decode launches take them in
// their arguments; routing and sparse attention read them from the tree's device geometry
// table instead (written by the build and append kernels), which keeps their arguments small.
struct ZLens {
  int32_t n[ZHA_MAX_BATCH];
};

struct zha_tree {
  zha_tree_desc desc;
  int device;
  int U, G, R, d, C, L, esize;
  int64_t T;                      // max_tokens (token stride of K/V)
  int64_t cap[ZHA_MAX_LEVELS + 2];  // nodes per unit at each level (1..L)
  int64_t span[ZHA_MAX_LEVELS + 2]; // tokens covered by one node at each level: C^l
  void* m[ZHA_MAX_LEVELS + 2];      // level planes m [U][cap][R][d] (tree dtype, or fp8 e4m3 codes)
  float* b[ZHA_MAX_LEVELS + 2];     // level planes b [U][cap][R]
  float* ms[ZHA_MAX_LEVELS + 2];    // fp8 summaries: power-of-two scale of each m row [U][cap][R];
                                    // fp4: scale bytes [U][cap][R][d/32] (else null)
  bool f8;                          // m stored as fp8 e4m3 codes
  bool f4;                          // m stored as fp4 e2m1 codes; ms holds a scale byte per block of 32
  int32_t* kept[ZHA_MAX_LEVELS + 2];// per-level kept ids [U][cap]
  unsigned long long* krank[ZHA_MAX_LEVELS + 2];  // union routes: per-level (stamp << 32) | rank in the
                                    // unit's kept list, by node id [RUmax][cap] (null: no union routes)
  uint32_t* route_ctr;              // [1] stamp of the current union route (advanced on the device)
  uint32_t* uflag;                  // union routes: [groups][kstride] stamp of each leaf chunk kept by
                                    // some routing unit of the union group
  int32_t* ulist;                   // [groups][cap1] those chunks in order (the group's level-1 kept list)
  int32_t* ucount;                  // [2][groups]: chunks in the list; chunks scanned
  int UGmax;                        // union groups the workspace is sized for
  bool uni_route;                   // the last route ran the union kernels
  float* refs;                      // [Hkv][R][d]
  float* spine;                     // [U][L+1] open-node accumulators (layout of the build path)
  int S;                            // subtree level of the build (highest level of <= 256 tokens)
  float* sub_lse;                   // [U][cap_S][R] fp32 LSE of finished level-S nodes (S < L only)
  float* sub_m;                     // [U][cap_S][R][d] fp32 means of finished level-S nodes
  int32_t* counts;                  // [2][L+2][U]: frontier counts, kept counts per level
  float* scores;                    // [U][cap1][G rounded up to 4] scores of a level of more than 1024 nodes
  float* sscore[2];                 // [U][1024][G rounded up to 4] scores of smaller levels, by level parity
  float* spart[2];                  // [U][WS][G][2] score-kernel partial log-sum-exp, by level parity
  uint32_t* keys;                   // [U][kstride] node-mass keys of the level being selected
  int64_t kstride;                  // cap1 rounded up to a multiple of 4
  uint32_t* fh_cnt;                 // [U][1024] fine mass histogram (zero between levels)
  unsigned long long* fh_mass;      // [U][1024]
  unsigned long long* fh_edge;      // [U][2]
  int32_t* cut;                     // [U][4] cut of the level being selected
  uint32_t* sel_cand;               // [U][min(32, 256/U)][8192][2] crossing-slice (key, position) pairs per selection workgroup
  uint32_t* sel_ctr;                // [U][1 + 32] selection workgroups arrived (zero between levels), candidates per workgroup
  unsigned long long* lb_status;    // [U][compaction chunks of level 1] look-back words
  uint32_t* lb_epoch;               // [RUmax][2] look-back epoch per unit (starts at 1), finished-workgroup count
  int32_t* lb_error;                // [1] set if a look-back wait ever gives up
  float* apart;                     // attention partials: o [U][WA][G][d], then (max, sum) [U][WA][G][2]
  int WS, WA;                       // score and attention workgroups per routing unit, last route's mode
  int hr;                           // routing units per (query, KV head) of the last route: 1 or G
  int Tq;                           // queries per sequence of the last route (1 unless multi-query)
  bool multi;                       // the last route was a multi-query route
  int RU;                           // routing units of the last route: U * Tq * hr
  int RUmax;                        // routing units the workspace is sized for: U * max_queries, times G
                                    // with per-head routes
  int32_t* geo;                     // [L+2][B] device: lengths (row 0), nodes of level l per sequence (row l)
  ZLens len;                        // current lengths
  ZLens len_prev;                   // lengths before the last zha_append
  bool built;
  uint64_t gen;                     // advanced by every zha_build and zha_append
  uint64_t route_gen;               // gen when the last route ran (attention needs it current)
  int64_t bytes;
  // timing
  int32_t timing_kernels;           // bit k: time launches of kernel code k (0: timing off)
  int32_t timing_levels;            // bit l: time launches at level l (bit 0: launches with no level)
  bool timing_open;                 // a begin event is recorded and waits for its end
  hipEvent_t ev[2 * ZHA_MAX_TIMING];
  int tk[ZHA_MAX_TIMING], tl[ZHA_MAX_TIMING];
  int n_rec;
};

// Timing helpers (record events around a launch when enabled).
void zha_time_begin(zha_tree* t, hipStream_t s, int kernel, int level);
void zha_time_end(zha_tree* t, hipStream_t s, int kernel, int level);

// Launchers (defined next to their kernels).  All return hipSuccess or the launch error.
hipError_t zha_launch_build(zha_tree* t, const void* K, hipStream_t s);
hipError_t zha_launch_append(zha_tree* t, const void* K, hipStream_t s);
hipError_t zha_launch_route(zha_tree* t, const void* q, float p, float scale, hipStream_t s);
hipError_t zha_launch_attend(zha_tree* t, const void* q, const void* K, const void* V, float scale,
                             float* out, float* lse, hipStream_t s);  // tail per t->multi
hipError_t zha_launch_dense(const void* q, const void* K, const void* V, const ZLens& len, int B, int Hq,
                            int Hkv, int d, int64_t T, zha_dtype dt, float scale, float* out, float* lse,
                            float* part, int WA, hipStream_t s);
hipError_t zha_launch_copy16(void* dst, const void* src, int64_t n16, hipStream_t s);
hipError_t zha_launch_decode_fp8(const uint8_t* codes, const float* scale, int64_t rows, int d, __bf16* out,
                                 hipStream_t s);
hipError_t zha_launch_decode_fp4(const uint8_t* codes, const uint8_t* scale, int64_t rows, int d, __bf16* out,
                                 float* scale_out, hipStream_t s);
int zha_sparse_wgs(int U);
int zha_score_wgs_units(int RU);  // score workgroups per routing unit (before the level's own cap)
// Union scoring of a route with Tq queries per sequence and hr units per (query, KV head):
// queries per group (0: no union scoring) and groups per (sequence, KV head).
int zha_union_queries(int R, int Gq, int Tq, int hr, bool wide);  // attention groups (64 query heads when
                                                                   // wide, i.e. bf16 K/V, else 16)
int zha_union_score_queries(int R, int Gq, int Tq, int hr);  // scoring groups (64 query heads)
int zha_dense_wgs(int U);
