// gfx950 kernels of libpkv and their C-ABI launchers: KV append, block copy,
// paged decode (split-K, fp16 or int8 K/V, optionally with shared-prefix
// work-groups), the log-sum-exp merge, and causal paged prefill.
//
// Paged decode follows the pages' statement of the problem: one new query
// token per sequence attends, softmax(q K^T / sqrt(d)) V ([p2]
// lqnn.cn/news/235768 §1.2), over every cached token, the one just appended
// included ([p2] §2.2 pseudocode); the cached K/V sit in fixed 16-token blocks
// reached through a per-sequence block table and are read in place, in table
// order, never gathered into contiguous memory ([p2] §3.2); several query heads
// share one KV head ([p1] chanyi.net.cn/article/49 §二, [p2] §4.2); the scores
// never go to HBM: each work-group runs a tiled online softmax over its part of
// the context, the Flash Attention idea of [p1] §四. Decode is bound by reading
// the cache ([p2] §1.3, §5.1), so the design target is HBM bandwidth, not
// arithmetic.
//
// Work decomposition (one work-group of 4 wave64s per (partition, KV head,
// sequence)):
//   * the partition's blocks are dealt round-robin to the 4 waves; each wave
//     streams its K and V tiles (16 rows x D) straight from HBM into VGPRs
//     with 16-byte loads, double-buffered so the next tile is in flight
//     while the current one is used; the loaded K tile serves all G query
//     heads of the group;
//   * scores on the matrix cores: one v_mfma_f32_16x16x32_f16 per 32 head
//     dims gives the G heads' scores of the tile's 16 tokens, each lane
//     receiving fully reduced scores of its token;
//   * softmax: base-2 online softmax with a wave-uniform running max that is
//     raised only when a score exceeds it by more than 8 (in log2 units), so
//     the rescale of the accumulators is a rare, wave-uniform branch;
//   * values: probabilities go through 256 bytes of LDS to a second lane
//     mapping in which each load instruction covers whole 256-byte rows and
//     each lane accumulates D/16 (fp16) output dims for all G heads;
//   * the 4 waves merge in LDS; a work-group writes one (m, l, o[D]) partial
//     per query head, or the final fp16 row when the sequence has a single
//     partition; a second kernel merges partitions by log-sum-exp.
// The reduction order depends only on logical token positions, so the result
// is bitwise independent of where the blocks live.
//
// With a shared-prefix plan, extra work-groups of the same launch attend the
// shared blocks of a group of sequences once for all their query rows
// (attend_rows, on the matrix cores); the paged prefill kernel runs the same
// multi-row attention, causally, for a chunk of new tokens.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <type_traits>
#include <cstdint>
#include <cstdlib>
#include <map>
#include <mutex>
#include <utility>

#include "pkv_internal.h"

namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int BT = PKV_BLOCK_TOKENS;  // tokens per block
constexpr int WAVES = 4;              // waves per decode work-group
constexpr float LAZY_MAX = 8.0f;      // rescale only when a score beats the max by 2^8
constexpr float LOG2E = 1.4426950408889634f;
// A wave keeps its tiles' block ids one per lane: at most 64 tiles per wave.
constexpr int MAX_PARTITION_TOKENS = 64 * WAVES * PKV_BLOCK_TOKENS;

// ---------------------------------------------------------------------------
// small device helpers

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float xor_shfl(float x, int mask) { return __shfl_xor(x, mask, 64); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load marked non-temporal: K/V tiles are read once per step, and
// streaming them without allocating in the caches sustains more HBM
// bandwidth on gfx950 than ordinary loads.
__device__ __forceinline__ uint4 load_nt(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Non-temporal for data read once (decode), cached for data re-read (prefill).
template <bool STREAM>
__device__ __forceinline__ uint4 load_tile(const void* p) {
  if constexpr (STREAM) return load_nt(p);
  const u32x4 v = *static_cast<const u32x4*>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float lo_half(uint32_t w) {
  return float(__builtin_bit_cast(half2_t, w).x);
}
__device__ __forceinline__ float hi_half(uint32_t w) {
  return float(__builtin_bit_cast(half2_t, w).y);
}

// Four int8 codes in one dword -> two fp16 pairs holding the exact integers.
// The bytes are biased to unsigned u = x + 128, placed in the low byte of
// fp16 1024 (whose ulp is 1) and the bias 1152 subtracted: exact for all
// codes.
__device__ __forceinline__ void i8x4_to_f16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
  const uint32_t u = w ^ 0x80808080u;
  const uint32_t a = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
  const uint32_t b = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
  const half2_t bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  lo = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, a) - bias);
  hi = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, b) - bias);
}

// Sixteen int8 codes (one 16-byte piece of a row) times their block's scale
// (both halves of s2), as sixteen fp16 values in two 16-byte pieces, in
// order. The codes are exact in fp16; the product is rounded once.
__device__ __forceinline__ void dequant16(const uint4& c, uint32_t s2, uint4& a, uint4& b) {
  const half2_t s = __builtin_bit_cast(half2_t, s2);
  uint32_t x[8];
  i8x4_to_f16x4(c.x, x[0], x[1]);
  i8x4_to_f16x4(c.y, x[2], x[3]);
  i8x4_to_f16x4(c.z, x[4], x[5]);
  i8x4_to_f16x4(c.w, x[6], x[7]);
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, x[k]) * s);
  a = make_uint4(x[0], x[1], x[2], x[3]);
  b = make_uint4(x[4], x[5], x[6], x[7]);
}

// The same codes biased by 1152: two halves holding 1152 + x, exact (no
// subtraction). Sums over biased codes are corrected once per head.
__device__ __forceinline__ void i8x4_to_f16x4_biased(uint32_t w, uint32_t& lo, uint32_t& hi) {
  const uint32_t u = w ^ 0x80808080u;
  lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
  hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
}

constexpr float I8_BIAS = 1152.0f;

// ---------------------------------------------------------------------------
// append / copy

// Token i, KV head h: copy the D-element rows k[i][h], v[i][h] into slot
// slots[i] of one layer. One thread moves 16 bytes.
__global__ __launch_bounds__(256) void append_kv_f16_kernel(uint4* __restrict__ Kl, uint4* __restrict__ Vl,
                                                            const uint4* __restrict__ k,
                                                            const uint4* __restrict__ v,
                                                            const int32_t* __restrict__ slots, int n,
                                                            int Hkv, int D, int num_blocks) {
  const int per_row = D / 8;  // 16-byte pieces per row
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = int64_t(n) * Hkv * per_row;
  if (idx >= total) return;
  const int c = int(idx % per_row);
  const int64_t th = idx / per_row;
  const int h = int(th % Hkv);
  const int64_t i = th / Hkv;
  const int32_t slot = slots[i];
  if (slot < 0 || slot >= num_blocks * BT) return;
  const int64_t blk = slot / BT, off = slot % BT;
  const int64_t dst = ((blk * Hkv + h) * BT + off) * per_row + c;
  const int64_t src = (i * Hkv + h) * per_row + c;
  Kl[dst] = k[src];
  Vl[dst] = v[src];
}

// int8 quantise-on-write of one fp16 row x into offset `off` of a (block,
// KV head) tile whose scale is sc, by one wave (lane l owns dims l + 64 e).
// With a = max |x| of the row:
//   offset 0:        s' = fp16(a / 127)           (the block is opened)
//   a <= 127 * s:    s' = s                       (the row fits the range)
//   otherwise:       s' = fp16(a / 127), and the earlier rows' codes are
//                    re-expressed: rint(code * s / s')
// then the row's codes are rint(x / s'), clipped to [-127, 127]; a zero
// scale gives zero codes. Divisions are IEEE fp32, rint rounds half to even.
// Each lane reads back only bytes it wrote itself. Returns s'.
template <int D>
__device__ __forceinline__ float quantise_row_i8(int8_t* tile, int off, const float (&x)[D / 64], float sc) {
  constexpr int PER = D / 64;  // dims per lane
  const int lane = threadIdx.x & 63;
  float a = 0.0f;
#pragma unroll
  for (int e = 0; e < PER; ++e) a = fmaxf(a, fabsf(x[e]));
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) a = fmaxf(a, xor_shfl(a, m));
  float sn = sc;
  bool requant = false;
  if (off == 0 || !(a <= 127.0f * sc)) {
    sn = float(_Float16(a / 127.0f));
    requant = off > 0;
  }
  if (requant) {
    for (int r = 0; r < off; ++r)
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        int8_t& c = tile[r * D + lane + 64 * e];
        c = sn == 0.0f ? int8_t(0) : int8_t(fminf(fmaxf(__builtin_rintf(float(c) * sc / sn), -127.0f), 127.0f));
      }
  }
#pragma unroll
  for (int e = 0; e < PER; ++e)
    tile[off * D + lane + 64 * e] =
        sn == 0.0f ? int8_t(0) : int8_t(fminf(fmaxf(__builtin_rintf(x[e] / sn), -127.0f), 127.0f));
  return sn;
}

// int8 append. One wave per (token i, KV head h, K or V); the wave whose
// token opens a run of consecutive tokens writing the same block appends the
// whole run in order (a block's scale depends on the order), each token by
// quantise_row_i8.
template <int D>
__global__ __launch_bounds__(64) void append_kv_i8_kernel(int8_t* __restrict__ Kl, int8_t* __restrict__ Vl,
                                                          _Float16* __restrict__ Sl,
                                                          const _Float16* __restrict__ k,
                                                          const _Float16* __restrict__ v,
                                                          const int32_t* __restrict__ slots, int n, int Hkv,
                                                          int num_blocks) {
  constexpr int PER = D / 64;  // dims per lane
  const int i = blockIdx.x, h = blockIdx.y, which = blockIdx.z;
  const int lane = threadIdx.x;
  const int nslots = num_blocks * BT;
  const int slot = slots[i];
  if (slot < 0 || slot >= nslots) return;
  const int blk = slot / BT;
  if (i > 0) {
    const int prev = slots[i - 1];
    if (prev >= 0 && prev < nslots && prev / BT == blk) return;  // inside a run led by an earlier wave
  }
  int8_t* tile = (which ? Vl : Kl) + (int64_t(blk) * Hkv + h) * BT * D;
  _Float16* sp = Sl + (int64_t(blk) * Hkv + h) * 2 + which;
  const _Float16* src = which ? v : k;
  float sc = float(*sp);
  for (int t = i; t < n; ++t) {
    const int sl = slots[t];
    if (t > i && (sl < 0 || sl >= nslots || sl / BT != blk)) break;
    float x[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) x[e] = float(src[(int64_t(t) * Hkv + h) * D + lane + 64 * e]);
    sc = quantise_row_i8<D>(tile, sl % BT, x, sc);
  }
  if (lane == 0) *sp = _Float16(sc);
}

// Copy-on-write: blockIdx = (pair, layer, region); region 0 = K, 1 = V,
// 2 = int8 scales. Copies the whole (layer, block) slab: Hkv tiles.
__global__ __launch_bounds__(256) void copy_blocks_kernel(char* __restrict__ pool, const int32_t* __restrict__ pairs,
                                                          int num_blocks, int64_t slab_bytes,
                                                          int64_t layer_bytes, int64_t region_bytes,
                                                          int64_t scale_slab_bytes, int has_scales) {
  const int pair = blockIdx.x, layer = blockIdx.y, region = blockIdx.z;
  const int32_t src = pairs[2 * pair], dst = pairs[2 * pair + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  if (region == 2) {
    if (!has_scales) return;
    const int64_t base = 2 * region_bytes + int64_t(layer) * num_blocks * scale_slab_bytes;
    const char* s = pool + base + src * scale_slab_bytes;
    char* d = pool + base + dst * scale_slab_bytes;
    for (int64_t i = threadIdx.x; i < scale_slab_bytes; i += blockDim.x) d[i] = s[i];
    return;
  }
  const int64_t base = region * region_bytes + layer * layer_bytes;
  const uint4* s = reinterpret_cast<const uint4*>(pool + base + src * slab_bytes);
  uint4* d = reinterpret_cast<uint4*>(pool + base + dst * slab_bytes);
  for (int64_t i = threadIdx.x; i < slab_bytes / 16; i += blockDim.x) d[i] = s[i];
}

// ---------------------------------------------------------------------------
// paged decode

struct DecodeParams {
  const void* K;  // this layer's K region: [N][Hkv][16][D]
  const void* V;
  const _Float16* scales;  // int8: this layer's [N][Hkv][2]; else null
  const _Float16* q;       // [B][Hq][D]
  const uint4* k_new;      // optional fused append: fp16 [B][Hkv][D] (null = none)
  const uint4* v_new;
  const int32_t* tables;
  const int32_t* ctx_lens;
  float* part_m;  // [B][Hq][max_parts]
  float* part_l;
  float* part_o;  // [B][Hq][max_parts][D]
  _Float16* out;  // [B][Hq][D]
  const int32_t* plan;  // shared-prefix plan (null = none): per sequence (shared blocks, group*64+member),
                        // then PKV_PREFIX_GROUP_INTS per group
  int prefix_z;         // grid z-planes of shared-prefix work-groups (0 = none)
  int plan_stream;      // plan grid: the split role is stream-K, its work-groups after the prefix ones
  int prefix_pp;        // prefix partitions per group
  int num_groups;
  int max_blocks;
  int num_blocks;
  int Hkv;
  int part_blocks;
  int max_parts;
  int max_context;
  float scale_log2;  // softmax scale * log2(e)
  int num_seqs;
  int stream_pad;    // stream-K split: blocks of start-up cost charged ahead of each sequence's span
  int group;         // query heads per KV head: the kernel's G, or fewer (its last heads are then padding)
};

__device__ __forceinline__ int clamp_ctx(int ctx, int max_blocks, int max_context) {
  return min(ctx, min(max_blocks * BT, max_context));
}

// Sequences a stream-K split can lay end to end (each work-group scans the
// partition counts of all of them).
constexpr int STREAM_MAX_SEQS = 1024;
// Start-up charge of a sequence's piece in a stream-K run, in blocks (int8
// blocks carry half the bytes, so twice as many). Measured on MI355X, split
// kernel us at a charge of 0 / 4 / 8 / 12 fp16 blocks (0 / 8 / 16 / 24
// int8): the continuous-batching mix 51.7 / 51.1 / 50.8 / 51.0, ragged int8
// 16 x U[128, 8192] (seed 7) 35.6 / 33.5 / 32.1 / 32.1; the shared-prefix
// launch 22.1 at every charge.
constexpr int STREAM_PAD_F16 = 8;
constexpr int STREAM_PAD_I8 = 16;

// Exclusive prefix sum of v over the 256 threads of a work-group (thread
// order), and the work-group's total. part: WAVES ints of LDS. Every thread
// must call it.
__device__ __forceinline__ int wg_exclusive_scan(int v, int* part, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) part[wave] = x;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) {
    const int t = part[w];
    off += w < wave ? t : 0;
    tot += t;
  }
  __syncthreads();  // part is rewritten by the next call
  total = tot;
  return off + x - v;
}

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

template <int D, int G, bool I8>
struct Shape {
  static constexpr int E = I8 ? 1 : 2;     // bytes per element
  static constexpr int NCH = D / 32;       // MFMA k-chunks of 32 dims
  static constexpr int KL = D * E / 64;    // K 16-byte loads per lane per tile
  static constexpr int CE = 16 / E;        // V elements per 16-byte chunk
  static constexpr int LPR = D / CE;       // V lanes per row
  static constexpr int RPI = 64 / LPR;     // V rows per load instruction
  static constexpr int NI = BT / RPI;      // V load instructions per tile
  static constexpr int TILE = BT * D * E;  // bytes per (block, head) tile
  // First of the 8 head dims that k-slot group j (lanes 16j..16j+15) holds in
  // MFMA chunk c. K load i of lane (n, j) reads bytes [16(4i + j), +16) of
  // row n: 8 fp16 dims (chunk i) or 16 int8 dims (chunks 2i and 2i + 1); q
  // is loaded with the same assignment, so the contraction pairs equal dims.
  static __device__ __forceinline__ int dim_base(int c, int j) {
    return I8 ? 64 * (c >> 1) + 16 * j + 8 * (c & 1) : 32 * c + 8 * j;
  }
};

// Max / sum over the 16 lanes of a DPP row. Every lane gets a result; lane 0
// of the row always combines in the same order.
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));   // quad_perm(1,0,3,2)
  x = fmaxf(x, dpp<0x4E>(x));   // quad_perm(2,3,0,1)
  x = fmaxf(x, dpp<0x124>(x));  // row_ror:4
  x = fmaxf(x, dpp<0x128>(x));  // row_ror:8
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x124>(x);
  x += dpp<0x128>(x);
  return x;
}
__device__ __forceinline__ float read_lane(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
// Entries 0..3 or 4..7 of an 8-entry per-head array, chosen by a flag that
// varies across lanes, as one select between two vector values (a select
// between two addresses in the array would move the array to scratch memory).
__device__ __forceinline__ float4_t half_of8(const float (&x)[8], bool upper) {
  const float4_t lo = {x[0], x[1], x[2], x[3]}, hi = {x[4], x[5], x[6], x[7]};
  return upper ? hi : lo;
}

// ---------------------------------------------------------------------------
// shared-prefix attention

// Query rows of a shared-prefix group per KV head: members x (Hq / Hkv), at
// most 128, attended by PREFIX_SPLIT work-groups of up to 64 rows (one
// 16-row MFMA block per wave).
constexpr int PREFIX_ROWS = 128;
constexpr int PREFIX_SPLIT = 2;
constexpr int PREFIX_HALF_ROWS = PREFIX_ROWS / PREFIX_SPLIT;

// A group's np shared blocks are cut into at most pp partitions of
// ceil(np / pp) blocks; prefix_parts of them are non-empty.
__device__ __forceinline__ int prefix_blocks_per_part(int np, int pp) { return (np + pp - 1) / pp; }
__device__ __forceinline__ int prefix_parts(int np, int pp) {
  if (np <= 0 || pp <= 0) return 0;
  const int pbp = prefix_blocks_per_part(np, pp);
  return (np + pbp - 1) / pbp;
}

// Shared blocks of sequence b and how many prefix partials lead its partial
// row (0 and 0 when it is in no group). The split kernel and the merge use
// this one rule.
__device__ __forceinline__ void seq_prefix(const int32_t* plan, int b, int max_blocks, int num_groups, int pp,
                                           int& sb, int& pre) {
  sb = 0;
  pre = 0;
  if (!plan) return;
  sb = min(max(plan[2 * b], 0), max_blocks);
  const int gm = plan[2 * b + 1];
  if (gm >= 0 && (gm >> 6) < num_groups && sb > 0) pre = prefix_parts(sb, pp);
}

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));

// 16 bytes per lane from global memory straight into LDS
// (global_load_lds_dwordx4): lane l reads base + ofs (base wave-uniform, in
// SGPRs, so the address costs no vector instruction; ofs the lane's 32-bit
// offset) and its bytes land at lds + 16 l (lds wave-uniform; checked on
// gfx950 with an in-bounds one-wave probe). Written as asm so that the
// compiler, which cannot tell which LDS bytes such a load writes, does not
// wait for every one in flight before each LDS read; the caller orders them
// itself: vmcnt waits (loads complete in order) before the barrier that
// hands the bytes to other waves, and before any reuse of the LDS. It has no
// register outputs; its operands are read at issue. The s_nop gives the
// five wait states a vector memory instruction needs after a VALU write of
// an SGPR it reads (and the one after the M0 write), whatever the compiler
// placed before the asm.
__device__ __forceinline__ void lds_load16(const char* base, uint32_t ofs, const char* lds) {
  const uint32_t m0 = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)lds));
  __asm__ __volatile__("s_mov_b32 m0, %0\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %1, %2"
                       :
                       : "s"(m0), "v"(ofs), "s"(base)
                       : "memory", "m0");
}

// Attention of up to 128 query rows over consecutive tiles of one block
// table, by a work-group of 4 waves on the matrix cores: the shared-prefix
// work-groups of the decode and the paged prefill both run it. Rows come in
// 16-row blocks (wave w takes blocks w and w + 4); row r's q is at qrow(r)
// (null: a padding row, never emitted). With MASK, row r sees logical
// tokens below limit(r) only (padding rows must not be masked entirely;
// every limit must be at least full_tokens, below which no row is masked),
// and V rows of tokens at or past nvalid (slots never written) are staged
// as zeros, so a masked weight of 0 never meets a stale NaN.
// Tiles jb .. jb + nt - 1 of `trow`, taken two at a time (a step of 32
// tokens). Their block ids sit in a ring of MAXT entries in LDS: the first
// MAXT are staged up front, and when nt exceeds MAXT the ring is refilled
// 256 ids at a time at a step barrier, each refill writing slots whose ids
// have already been read. STREAM: tiles are read
// once (non-temporal loads); otherwise other work-groups re-read them, and
// ordinary loads keep them in L2. emit(r, o, m, l)
// receives row r's unnormalised output, lane (n, j) holding dims
// 16 i + 4 j + e of row 16 rb + n, with the row's base-2 running max m and
// its sum l.
//
// Per step and row block:
//   S^T (16 tokens x 16 rows) = K (16 x D) . Q^T (D x 16) for each of the
//       two tiles, v_mfma_f32_16x16x32_f16 over D/32 chunks: lane (n, j)
//       receives tokens 4j..4j+3 of query row n from each tile;
//   O^T (D x 16 rows) += V^T (D x 32 tokens) . P^T (32 tokens x 16 rows),
//       one v_mfma_f32_16x16x32_f16 per 16 dims. The contraction's k slots
//       8j..8j+7 of lane (n, j) are tokens 4j..4j+3 of the first tile and
//       then of the second: exactly the scores the lane holds, so P goes from
//       one MFMA to the next without moving between lanes.
// K and V tiles are both staged in LDS row-major: padded rows written from
// a register ring of loads, or (the DMA mode below) unpadded, swizzled rows
// loaded straight into LDS. The V^T operand comes from the LDS transpose read
// ds_read_b64_tr_b16: within each 16-lane group, lane s addresses 4
// halves and lane i receives element i % 4 of lanes i/4, 4 + i/4, 8 + i/4
// and 12 + i/4 (checked on gfx950 with a one-wave probe). With lane s of
// group j pointing at V[4j + s/4][16 i + 4 (s % 4)], lane (n, j) receives
// V[4j..4j+3][16 i + n]: the A operand, 4 tokens of one dim. Online
// softmax per row in base 2 with the lazy running max of the split kernel.
template <int D, int MAXT, bool MASK, bool STREAM, int PFS, bool I8, int RB, typename QRow, typename Limit,
          typename Emit>
__device__ __forceinline__ void attend_rows(const char* Kc, const char* Vc, const uint32_t* scales, int Hkv, int g,
                                            int num_blocks, const int32_t* trow, int jb, int nt, int R, int nvalid,
                                            int full_tokens, float scale_log2, QRow qrow, Limit limit,
                                            Emit emit) {
  constexpr int NCH = D / 32;           // score MFMA chunks
  constexpr int NDB = D / 16;           // value MFMA dim blocks
  constexpr int KROW = D * 2 + 16;      // bytes per staged K row (16 lanes read 16 rows without conflicts)
  constexpr int VROW = D * 2 + 32;      // bytes per staged V row (the transpose read's 4-row groups
                                        // start 8 banks apart)
  constexpr int E = I8 ? 1 : 2;         // bytes per element in the pool
  constexpr int PIECES = D * E / 16;    // 16-byte pieces per K/V row in the pool
  constexpr int LOADERS = BT * PIECES;  // pieces per K (or V) tile
  constexpr int TILE = BT * D * E;      // pool bytes per (block, KV head) tile
  // PFS: steps (tile pairs) in flight per thread
  static_assert(PFS % 2 == 0, "LDS stages alternate with the ring slot");
  // DMA (fp16 d128, two row blocks per wave: the paged prefill): tiles go
  // from HBM straight into LDS (global_load_lds, 16 bytes per lane), three
  // stages of a step's two K and two V tiles,
  // unpadded, each row's 16-byte pieces XOR-swizzled by the row index so
  // that 16 lanes reading one piece of 16 rows (K) or 4 rows (the V
  // transpose read) hit distinct banks. Otherwise tiles are loaded into a
  // register ring and stored to two padded LDS stages.
  constexpr bool DMA = !I8 && D == 128 && RB == 2;
  constexpr int TB = BT * D * 2;  // bytes per staged fp16 tile
  __shared__ __align__(16) char dma_st[DMA ? 3 : 1][DMA ? 4 * TB : 16];
  __shared__ __align__(16) char kst[DMA ? 1 : 2][2][DMA ? 16 : BT * KROW];
  __shared__ __align__(16) char vst[DMA ? 1 : 2][2][DMA ? 16 : BT * VROW];
  __shared__ int blk_ids[MAXT];
  __shared__ uint32_t tile_sc[I8 ? MAXT : 1];  // int8: each tile's (K, V) fp16 scales
  constexpr int REFILL = 256;  // ids per refill: one per thread
  static_assert(MAXT > REFILL || MAXT <= 64, "a refilled ring must hold more than one refill");

  const int tid = threadIdx.x, lane = tid & 63;
  __builtin_assume(tid < 256);  // work-groups of 256 threads
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 15, lj = lane >> 4;
  auto stage_id = [&](int i) {  // tile i's id (and int8 scales) into its ring slot
    const int blk = trow[jb + i];
    blk_ids[i % MAXT] = blk;
    if constexpr (I8) tile_sc[i % MAXT] = unsigned(blk) < unsigned(num_blocks) ? scales[int64_t(blk) * Hkv + g] : 0u;
  };
  for (int i = tid; i < min(nt, MAXT); i += 256) stage_id(i);
  // After the loads of step it + 1 + PFS are issued, every tile below
  // T0 = 2 (it + 2 + PFS) has been read; when T0 is a multiple of REFILL, the
  // slots of tiles T0 - REFILL .. T0 - 1 take tiles MAXT further on, first
  // read (MAXT - REFILL) / 2 steps later, after the barrier that ends this
  // step. Uniform over the work-group; never taken when nt <= MAXT.
  auto refill = [&](int it) {
    const int T0 = 2 * (it + (DMA ? 3 : 2 + PFS));  // DMA: the loads of step it + 2 are issued
    if (T0 % REFILL == 0 && T0 - REFILL + MAXT < nt) {
      const int t = T0 - REFILL + MAXT + tid;
      if (t < nt) stage_id(t);
    }
  };
  const int nsteps = (nt + 1) / 2;

  // q^T as the B operand of the score MFMA, per row block of this wave. A
  // negative scale's sign moves into q (exact), so the scores below are
  // always multiplied by sl2 = |scale_log2|: a raw score a then exceeds the
  // threshold thr = (m + LAZY_MAX) / sl2 exactly when its scaled value beats
  // the running max m by more than LAZY_MAX.
  static_assert(RB == 1 || RB == 2, "one or two 16-row blocks per wave");
  const int rb0 = wave, rb1 = wave + 4;
  const bool has0 = rb0 * 16 < R, has1 = RB == 2 && rb1 * 16 < R;
  const uint32_t qsign = scale_log2 < 0.0f ? 0x80008000u : 0u;
  const float sl2 = fabsf(scale_log2), inv_sl2 = 1.0f / sl2;
  auto load_q = [&](int rb, half8_t (&qb)[NCH]) {
    const _Float16* qp = qrow(rb * 16 + ln);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      u32x4 w = qp ? *reinterpret_cast<const u32x4*>(qp + 32 * c + 8 * lj) : u32x4{0u, 0u, 0u, 0u};
      w ^= qsign;
      qb[c] = __builtin_bit_cast(half8_t, w);
    }
  };
  half8_t q0[NCH], q1[NCH];
  load_q(rb0, q0);
  if constexpr (RB == 2) load_q(rb1, q1);
  const int lim0 = MASK ? limit(rb0 * 16 + ln) : 0, lim1 = MASK ? limit(rb1 * 16 + ln) : 0;

  float4_t o0[NDB], o1[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    o0[i] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    o1[i] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }
  float m0 = -INFINITY, m1 = -INFINITY, l0 = 0.0f, l1 = 0.0f, thr0 = -INFINITY, thr1 = -INFINITY;
  // DMA mode: the row sums on the matrix cores, P^T against an all-ones
  // operand (every element of ls is the row's sum); otherwise v_dot2 sums
  // per lane, reduced over the four token groups at the end
  float4_t ls0 = {0.0f, 0.0f, 0.0f, 0.0f}, ls1 = {0.0f, 0.0f, 0.0f, 0.0f};
  half8_t ones8 = {(_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f,
                   (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f};
  // held in registers for the whole walk: the compiler would otherwise
  // rebuild it every step (two vector moves)
  if constexpr (DMA) __asm__("" : "+v"(ones8));

  // Tile staging: a tile is 2 x LOADERS 16-byte pieces (K, then V), each
  // piece along a row; thread t moves pieces t + 256 j (int8 at D = 64: only
  // threads below 2 x LOADERS). Steps are fetched PFS ahead into a register
  // ring; the loads are unconditional (tiles past the last re-read it) so the
  // compiler counts outstanding loads statically. int8 pieces are
  // dequantised with their tile's scale as they are stored, so LDS always
  // holds fp16.
  constexpr int NLD = (2 * LOADERS + 255) / 256;
  uint4 ring[PFS][2][NLD];
  auto piece = [&](int q, int& lrow, int& lpc) {
    const int pc = q % LOADERS;
    lrow = pc / PIECES;
    lpc = pc % PIECES;
  };
  // Block id of tile t (past the last tile: the last tile's) for the loads.
  // The ids of 64 consecutive tiles (wb .. wb + 63) sit one per lane in idw
  // and are taken with readlane, so the loads of a step wait for no LDS read
  // of their ids; idw is refreshed from the ring every 32 steps (tiles only
  // grow, and those read are staged long before).
  int wb = -64, idw = -1;
  auto tile_block = [&](int t) {
    t = min(t, nt - 1);
    if (t >= wb + 64) {  // wave-uniform
      wb = t & ~63;
      idw = blk_ids[(wb + lane) % MAXT];
    }
    return __builtin_amdgcn_readlane(idw, t - wb);
  };
  auto gload = [&](int step, uint4 (&r)[2][NLD]) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int blk = tile_block(2 * step + sub);
      const int safe = unsigned(blk) < unsigned(num_blocks) ? blk : 0;
      const int64_t base = (int64_t(safe) * Hkv + g) * TILE;
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        const int q = tid + 256 * j;
        if (I8 && q >= 2 * LOADERS) continue;  // int8 at D = 64 only; uniform per wave
        int lrow, lpc;
        piece(q, lrow, lpc);
        r[sub][j] = load_tile<STREAM>((q < LOADERS ? Kc : Vc) + base + lrow * (D * E) + lpc * 16);
      }
    }
  };
  auto lstore = [&](int st, const uint4 (&r)[2][NLD], int step) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        const int q = tid + 256 * j;
        int lrow, lpc;
        // V rows at or past nvalid of this tile: `room` of its rows are
        // valid, all of them unless it holds the end of the written tokens
        // (a uniform test, so whole tiles skip the per-row one)
        const int room = nvalid - (jb + 2 * step + sub) * BT;
        if constexpr (I8) {
          if (q >= 2 * LOADERS) continue;
          piece(q, lrow, lpc);
          const bool live = q < LOADERS || !MASK || room >= BT || lrow < room;
          char* dst = q < LOADERS ? kst[st][sub] + lrow * KROW : vst[st][sub] + lrow * VROW;
          const uint32_t sc = tile_sc[min(2 * step + sub, nt - 1) % MAXT];
          const uint32_t s1 = q < LOADERS ? (sc & 0xffffu) : (sc >> 16);  // K or V scale
          uint4 a, b;
          dequant16(r[sub][j], s1 | (s1 << 16), a, b);
          *reinterpret_cast<uint4*>(dst + lpc * 32) = live ? a : make_uint4(0u, 0u, 0u, 0u);
          *reinterpret_cast<uint4*>(dst + lpc * 32 + 16) = live ? b : make_uint4(0u, 0u, 0u, 0u);
        } else {
          piece(q, lrow, lpc);
          if (q < LOADERS) {
            *reinterpret_cast<uint4*>(kst[st][sub] + lrow * KROW + lpc * 16) = r[sub][j];
          } else {
            uint4* dst = reinterpret_cast<uint4*>(vst[st][sub] + lrow * VROW + lpc * 16);
            *dst = r[sub][j];
            if (MASK && room < BT && lrow >= room) *dst = make_uint4(0u, 0u, 0u, 0u);  // same lane: in order
          }
        }
      }
    }
  };

  // DMA staging: lane l of wave w moves row 4 w + l / 16 of a tile, its
  // 16 bytes landing at LDS slot l % 16 of that row; it loads the tile's
  // piece (l % 16) ^ row, so slot s of row r holds piece s ^ r.
  const int drow = 4 * wave + (lane >> 4);
  const int dofs = drow * (D * 2) + (((lane & 15) ^ drow) << 4);
  auto dma_tile = [&](int st, int k) { return dma_st[st] + k * TB; };  // k: K0, K1, V0, V1
  auto dma_step = [&](int st, int step) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int blk = tile_block(2 * step + sub);
      const int safe = unsigned(blk) < unsigned(num_blocks) ? blk : 0;
      const int64_t base = (int64_t(safe) * Hkv + g) * TILE;
      lds_load16(Kc + base, dofs, dma_tile(st, sub) + 1024 * wave);
      lds_load16(Vc + base, dofs, dma_tile(st, 2 + sub) + 1024 * wave);
    }
  };
  // after this wave's loads of `step` have landed: V rows at or past nvalid
  // in the tile that holds the end of the written tokens become zeros
  // (each lane rewrites the 16 bytes its own load wrote). The step test is
  // uniform (a scalar branch), so steps before the end cost no vector
  // instruction.
  auto dma_zero_tail = [&](int st, int step) {
    if constexpr (MASK) {
      if ((jb + 2 * step + 2) * BT > nvalid) {
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          const int room = nvalid - (jb + 2 * step + sub) * BT;
          if (drow >= room)
            *reinterpret_cast<uint4*>(dma_tile(st, 2 + sub) + 1024 * wave + 16 * lane) = make_uint4(0u, 0u, 0u, 0u);
        }
      }
    }
  };
  // wait until at most n of this wave's vector-memory loads are in flight
  // (loads complete in order); vmcnt(n), expcnt and lgkmcnt not waited on
  auto wait_loads = [](auto n) {
    static_assert(decltype(n)::value >= 0 && decltype(n)::value < 16, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt(0x0F70 | decltype(n)::value);
  };
  // The step barrier of the DMA loop: this wave's LDS accesses done
  // (lgkmcnt(0)) and all but the newest step's four tile loads landed
  // (vmcnt(4)), then s_barrier. A __syncthreads() would also wait for the
  // newest loads (its work-group fence covers the LDS they write), which
  // would leave no load in flight across the barrier. The empty asm keeps
  // the compiler from moving memory accesses across it.
  auto dma_barrier = []() {
    __builtin_amdgcn_s_waitcnt(0x0074);
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ __volatile__("" ::: "memory");
  };

  // Online softmax of one row block's scores of a step (two tiles), kept
  // short because the VALU, not the matrix cores, sets this loop's pace, and
  // split in two so the exponentials of one row block can issue beside the
  // other's value MFMAs. prep: masking only in the `masked` variant (the
  // diagonal and the odd tail, chosen per step) and the lazy-max test, one
  // compare per raw score against the row's threshold (raising m, thr and
  // rescaling when any lane's score passes it). probs: one FMA into each
  // exponential, row sums of the fp16 probabilities by v_dot2 against ones;
  // returns P in the value MFMA's k-slot order.
  auto prep = [&](const float4_t (&acc)[2], int step, int lim, auto masked, float4_t (&o)[NDB], float& m,
                  float& l, float& thr, float4_t& ls, float (&a)[8]) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int e = 0; e < 4; ++e) a[sub * 4 + e] = acc[sub][e];
    if constexpr (decltype(masked)::value) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const int tile = 2 * step + sub;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool out = tile >= nt || (MASK && (jb + tile) * BT + 4 * lj + e >= lim);
          a[sub * 4 + e] = out ? -INFINITY : a[sub * 4 + e];
        }
      }
    }
    bool up = false;
#pragma unroll
    for (int k = 0; k < 8; ++k) up |= a[k] > thr;
    if (__builtin_amdgcn_ballot_w64(up)) {  // wave-uniform, rare after the first step
      const float amax =
          fmaxf(fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3])), fmaxf(fmaxf(a[4], a[5]), fmaxf(a[6], a[7])));
      float mx = amax * sl2;
      mx = fmaxf(mx, xor_shfl(mx, 16));
      mx = fmaxf(mx, xor_shfl(mx, 32));
      const float mn = fmaxf(m, mx);
      const float alpha = (m == -INFINITY) ? 0.0f : exp2_fast(m - mn);
      m = mn;
      thr = (m + LAZY_MAX) * inv_sl2;
      if constexpr (DMA)
        ls *= alpha;
      else
        l *= alpha;
#pragma unroll
      for (int i = 0; i < NDB; ++i) o[i] *= alpha;
    }
  };
  // probabilities enter the value MFMA in fp16; the row sum adds the same
  // rounded values, so weights and normaliser agree
  auto probs = [&](const float (&a)[8], float m, float& l) {
    const float nm = -m;
    half2_t pp[4];
    const half2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      pp[k] = half2_t{(_Float16)exp2_fast(__builtin_fmaf(a[2 * k], sl2, nm)),
                      (_Float16)exp2_fast(__builtin_fmaf(a[2 * k + 1], sl2, nm))};
      if constexpr (!DMA) l = __builtin_amdgcn_fdot2(pp[k], ones, l, false);
    }
    return __builtin_bit_cast(half8_t, pp);
  };

  // One step for both row blocks of the wave: every K and V fragment is
  // read from LDS once and used by both. Both blocks are always computed
  // (rows past R have zero q and are never emitted): guards around single
  // MFMAs would become branches that split the scheduling regions. After
  // both prep branches the remaining work is one region, ordered so the
  // second block's exponentials sit between the first block's value MFMAs.
  auto step_rows = [&](int st, int step, auto masked) {
    float4_t acc0[2], acc1[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      acc0[sub] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
      acc1[sub] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const char* kp = DMA ? dma_tile(st, sub) + ln * (D * 2) + (((4 * c + lj) ^ ln) << 4)
                             : kst[DMA ? 0 : st][sub] + ln * KROW + (32 * c + 8 * lj) * 2;
        const half8_t ka = *reinterpret_cast<const half8_t*>(kp);
        acc0[sub] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, q0[c], acc0[sub], 0, 0, 0);
        if constexpr (RB == 2) acc1[sub] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, q1[c], acc1[sub], 0, 0, 0);
      }
    }
    float a0[8], a1[8];
    prep(acc0, step, lim0, masked, o0, m0, l0, thr0, ls0, a0);
    if constexpr (RB == 2) prep(acc1, step, lim1, masked, o1, m1, l1, thr1, ls1, a1);
    const half8_t pt0 = probs(a0, m0, l0);
    if constexpr (DMA) {
      // lane (n, j) addresses V[4j + n/4][16 i + 4 (n % 4)] of each tile:
      // piece 2 i + (n % 4) / 2 of row 4j + n/4, half (n % 2) of it; both
      // row blocks' probabilities first, so each V fragment is used by the
      // two MFMAs right after its read (no registers hold all of them)
      const half8_t pt1 = RB == 2 ? probs(a1, m1, l1) : pt0;
      const int vr = 4 * lj + (ln >> 2);
#pragma unroll
      for (int i = 0; i < NDB; ++i) {
        const int vofs = vr * (D * 2) + (((2 * i + ((ln >> 1) & 1)) ^ vr) << 4) + 8 * (ln & 1);
        const short4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) short4_t*)(dma_tile(st, 2) + vofs));
        const short4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) short4_t*)(dma_tile(st, 3) + vofs));
        const half8_t va = __builtin_bit_cast(half8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        o0[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pt0, o0[i], 0, 0, 0);
        if constexpr (RB == 2) o1[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pt1, o1[i], 0, 0, 0);
      }
      ls0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones8, pt0, ls0, 0, 0, 0);
      if constexpr (RB == 2) ls1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones8, pt1, ls1, 0, 0, 0);
      return;
    }
    // lane (n, j) addresses V[4j + n/4][16 i + 4 (n % 4)] of each tile
    const int vofs = (4 * lj + (ln >> 2)) * VROW + (ln & 3) * 8;
    half8_t va[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) {
      const short4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) short4_t*)(vst[DMA ? 0 : st][0] + vofs + 32 * i));
      const short4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) short4_t*)(vst[DMA ? 0 : st][1] + vofs + 32 * i));
      va[i] = __builtin_bit_cast(half8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      o0[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[i], pt0, o0[i], 0, 0, 0);
    }
    if constexpr (RB == 2) {
      const half8_t pt1 = probs(a1, m1, l1);
#pragma unroll
      for (int i = 0; i < NDB; ++i) o1[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[i], pt1, o1[i], 0, 0, 0);
    }
    // interleave: one MFMA, then a few VALU instructions, while they last
    if constexpr (RB == 2) {
#pragma unroll
      for (int i = 0; i < NDB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
    }
  };

  // steps with both tiles real and every token visible to every row
  int nfree = nt / 2;
  if (MASK) nfree = min(nfree, max(0, (full_tokens / BT - jb) / 2));

  __syncthreads();  // block ids
  if constexpr (DMA) {
    // Step s sits in LDS stage s % 3. Iteration it: the math of step it
    // (stage it % 3), the loads of step it + 2 into stage (it + 2) % 3 --
    // last read in iteration it - 1, which a barrier ended -- and, once this
    // wave's loads of step it + 1 have landed (only step it + 2's four may
    // still be in flight), the barrier that hands stage (it + 1) % 3 to all
    // waves. A loop runs rounds of three steps (unrolled, so every stage is
    // a constant); past its last step only the math is skipped.
    dma_step(0, 0);
    dma_step(1, 1);
    wait_loads(std::integral_constant<int, 4>{});
    dma_zero_tail(0, 0);
    dma_barrier();
    auto run3 = [&](int from, int to, auto masked) {
      for (int it0 = from; it0 < to; it0 += 3) {
#pragma unroll
        for (int u = 0; u < 3; ++u) {
          const int it = it0 + u;
          if (it < to) step_rows(u, it, masked);
          dma_step((u + 2) % 3, it + 2);
          refill(it);
          wait_loads(std::integral_constant<int, 4>{});
          dma_zero_tail((u + 1) % 3, it + 1);
          dma_barrier();
        }
      }
    };
    nfree -= nfree % 3;
    run3(0, nfree, std::false_type{});
    run3(nfree, nsteps, std::true_type{});
    wait_loads(std::integral_constant<int, 0>{});  // the last loads (past the end) land before the LDS is reused
  } else {
#pragma unroll
  for (int u = 0; u < PFS; ++u) gload(u, ring[u]);
  lstore(0, ring[0], 0);
  gload(PFS, ring[0]);
  __syncthreads();
  // Step it sits in LDS stage it & 1 and its successor in ring slot
  // (it + 1) % PFS. A loop runs whole rounds of PFS (unrolled, so every slot
  // index is a constant); past its last step only the math is skipped:
  // loads and stores stay unconditional, and the compiler's count of loads
  // in flight stays exact across the loop. Two loops: the leading steps no
  // row masks (whole rounds of them), then the rest with masks (the
  // diagonal and the odd tail); separate loops keep the two variants'
  // registers apart.
  auto run = [&](int from, int to, auto masked) {
    for (int it0 = from; it0 < to; it0 += PFS) {
#pragma unroll
      for (int u = 0; u < PFS; ++u) {
        const int it = it0 + u;
        const int st = u & 1;  // == it & 1: `from` and PFS are even
        if (it < to) step_rows(st, it, masked);
        lstore(st ^ 1, ring[(u + 1) % PFS], it + 1);
        gload(it + 1 + PFS, ring[(u + 1) % PFS]);
        refill(it);
        __syncthreads();
      }
    }
  };
  nfree -= nfree % PFS;
  run(0, nfree, std::false_type{});
  run(nfree, nsteps, std::true_type{});
  }

  // the row sums over the four token groups
  if constexpr (DMA) {
    l0 = ls0[0];
    l1 = ls1[0];
  } else {
    l0 += xor_shfl(l0, 16);
    l0 += xor_shfl(l0, 32);
    if constexpr (RB == 2) {
      l1 += xor_shfl(l1, 16);
      l1 += xor_shfl(l1, 32);
    }
  }
  if (has0 && rb0 * 16 + ln < R) emit(rb0 * 16 + ln, o0, m0, l0);
  if constexpr (RB == 2)
    if (has1 && rb1 * 16 + ln < R) emit(rb1 * 16 + ln, o1, m1, l1);
}

// The shared-prefix role of a decode work-group: KV head g, partition `part`
// of group grp's shared blocks, query rows half * 64 .. half * 64 + 63 of the
// group's (two work-groups share a partition's rows: each step's chain of
// matrix and softmax work is half as long, and the second reads the tiles
// the first brought into its XCD's L2, the two being PREFIX_SPLIT apart in
// dispatch order, Hkv work-groups apart in linear id). The group's members share their leading
// blocks ([p1] §三): each K/V tile of the run is read once here and attended
// by all R = members x G query rows. Shared blocks are full, so nothing is
// masked. Each row ends as one (m, l, o[D]) partial, written into slot
// `part` of the member's own partial row, ahead of its split-K partials.
template <int D, int G, bool I8>
__device__ __forceinline__ void prefix_role(const DecodeParams& prm, int g, int grp, int part, int half) {
  constexpr int NDB = D / 16;
  const int lj = (threadIdx.x & 63) >> 4;
  const int B = prm.num_seqs, gr = prm.group, Hq = prm.Hkv * gr;  // rows: (member, head of the group)
  const int32_t* gd = prm.plan + 2 * int64_t(B) + int64_t(grp) * PKV_PREFIX_GROUP_INTS;
  const int np = min(gd[0], prm.max_blocks);
  const int members = min(gd[1], PKV_MAX_SHARERS);
  const int R = min(members * gr, PREFIX_ROWS);
  const int r0 = half * PREFIX_HALF_ROWS;  // this work-group's rows: r0 .. r0 + 63 of the group's
  const int Rh = min(R - r0, PREFIX_HALF_ROWS);
  const int b0 = gd[2];
  if (np <= 0 || Rh <= 0 || unsigned(b0) >= unsigned(B)) return;
  const int pbp = prefix_blocks_per_part(np, prm.prefix_pp);  // <= 64: the host sizes prefix_pp
  const int jb = part * pbp, je = min(np, jb + pbp);
  if (jb >= je) return;
  auto member_of = [&](int r) { return r < Rh ? gd[2 + (r0 + r) / gr] : -1; };
  auto qrow = [&](int r) -> const _Float16* {
    const int bb = member_of(r);
    return unsigned(bb) < unsigned(B) ? prm.q + (int64_t(bb) * Hq + g * gr + (r0 + r) % gr) * D : nullptr;
  };
  auto no_limit = [](int) { return 0; };
  auto emit = [&](int r, const float4_t (&o)[NDB], float m, float l) {
    const int bb = member_of(r);
    if (unsigned(bb) >= unsigned(B)) return;
    const int64_t pi = (int64_t(bb) * Hq + g * gr + (r0 + r) % gr) * prm.max_parts + part;
#pragma unroll
    for (int i = 0; i < NDB; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) prm.part_o[pi * D + 16 * i + 4 * lj + e] = o[i][e];
    if (lj == 0) {
      prm.part_m[pi] = m;
      prm.part_l[pi] = l;
    }
  };
  attend_rows<D, 64, false, false, 2, I8, 1>(static_cast<const char*>(prm.K), static_cast<const char*>(prm.V),
                                         reinterpret_cast<const uint32_t*>(prm.scales), prm.Hkv, g, prm.num_blocks,
                                         prm.tables + int64_t(b0) * prm.max_blocks, jb, je - jb, Rh, 0, 0,
                                         prm.scale_log2, qrow, no_limit, emit);
}

// ---------------------------------------------------------------------------
// paged prefill

// Block ids a prefill work-group keeps in LDS at once (a ring: longer
// contexts are refilled as the walk proceeds).
constexpr int PREFILL_MAX_TILES = 1024;
// Steps (pairs of tiles) a prefill work-group keeps in flight.
constexpr int PREFILL_PFS = 2;

struct PrefillParams {
  const char* K;  // this layer's K region: [N][Hkv][16][D] fp16
  const char* V;
  const _Float16* q;        // [T][Hq][D], sequence-major
  const int32_t* q_start;   // [B + 1]: sequence b's rows q_start[b] .. q_start[b + 1] - 1
  const int32_t* tables;    // [B][max_blocks]
  const int32_t* ctx_lens;  // [B]: cached tokens, the chunk's own included
  _Float16* out;            // [T][Hq][D]
  const uint32_t* scales;   // int8: this layer's (K, V) fp16 scales [N][Hkv]; else null
  int Hkv, max_blocks, num_blocks, max_context;
  float scale_log2;
  int group;  // query heads per KV head (the kernel's G when it has one)
};

// Causal attention of a chunk of new tokens over the paged cache ([p1] §二
// and [p2] §1.3: the prompt's tokens are processed together; [p1] §四: tiled
// with an online softmax, same result). A query tile is 128 / G consecutive
// tokens of a sequence's chunk, and its rows are (token, query head of the
// group), so every K/V tile read is attended by 128 query rows on the
// matrix cores. Token i of sequence b's chunk sits at logical position
// ctx - qlen + i and sees tokens 0..itself; a query tile walks K/V tiles 0 ..
// that of its last token, masking per row. Causal tiles differ in length
// (the last walks the whole context, the first its prefix only), so each
// work-group (KV head g, pair y, sequence b) takes two of them, the
// sequence's tile Q - 1 - y and then tile y (Q tiles in all; the middle one
// alone when Q is odd): every pair walks about the same number of steps, and
// one round of work-groups holds no long tile that would run on after the
// others have drained.
template <int D, int G, bool I8>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillParams prm) {
  constexpr int NDB = D / 16;
  const int gr = G > 0 ? G : prm.group;  // G = 0: any group size, taken at run time
  const int QT = PREFIX_ROWS / gr;       // query tokens per tile
  const int g = blockIdx.x, y = blockIdx.y, b = blockIdx.z;
  const int Hq = prm.Hkv * gr;
  const int t0 = prm.q_start[b], ql = prm.q_start[b + 1] - t0;
  const int n = clamp_ctx(prm.ctx_lens[b], prm.max_blocks, prm.max_context);
  if (ql <= 0 || ql > n) return;
  const int Q = (ql + QT - 1) / QT;
  if (2 * y >= Q) return;
  const int lj = (threadIdx.x & 63) >> 4;
  const int passes = 2 * y + 1 < Q ? 2 : 1;
  for (int pass = 0; pass < passes; ++pass) {
    const int i0 = (pass == 0 ? Q - 1 - y : y) * QT;
    const int cnt = min(QT, ql - i0), R = cnt * gr;
    const int pos0 = n - ql + i0;  // logical position of the tile's first token
    const int nt = (pos0 + cnt - 1) / BT + 1;
    auto qrow = [&](int r) -> const _Float16* {
      return r < R ? prm.q + (int64_t(t0 + i0 + r / gr) * Hq + g * gr + r % gr) * D : nullptr;
    };
    auto limit = [&](int r) { return r < R ? pos0 + r / gr + 1 : INT_MAX; };
    auto emit = [&](int r, const float4_t (&o)[NDB], float, float l) {
      _Float16* dst = prm.out + (int64_t(t0 + i0 + r / gr) * Hq + g * gr + r % gr) * D + 4 * lj;
      const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
      for (int i = 0; i < NDB; ++i) {
        half4_t h;
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = (_Float16)(o[i][e] * inv);
        *reinterpret_cast<half4_t*>(dst + 16 * i) = h;
      }
    };
    if (pass) __syncthreads();  // the first walk's LDS reads are done
    attend_rows<D, PREFILL_MAX_TILES, true, false, PREFILL_PFS, I8, 2>(prm.K, prm.V, prm.scales, prm.Hkv, g,
                                                                    prm.num_blocks,
                                                                    prm.tables + int64_t(b) * prm.max_blocks, 0, nt,
                                                                    R, n, pos0 + 1, prm.scale_log2, qrow, limit, emit);
  }
}

// ---------------------------------------------------------------------------
// int8 decode stream: both products on the matrix cores

// One wave's stream over its int8 tiles (logical blocks first, first + 4,
// ..., n_my of them; block ids one per lane in blk_lane), two tiles per step:
//   * scores S^T (16 tokens x 16 rows) = K (16 x D) . Q^T (D x 16) per tile,
//     v_mfma_f32_16x16x32_f16 over D/32 chunks, with the codes entering as
//     fp16 1152 + x (exact; the term 1152 * sum_d q[h][d] is removed from
//     every score of head h). Row r of Q^T is query head r % G of the group,
//     so rows repeat when G < 16; lane (n, j) receives tokens 4j..4j+3 of
//     row n, and every lane works on the single head n % G;
//   * base-2 online softmax per row, the running max raised only when a
//     score beats it by more than 2^8 (a rare, wave-uniform branch);
//   * values O^T (D x 16 rows) += V^T (D x 32 tokens) . P^T (32 tokens x 16
//     rows), one v_mfma_f32_16x16x32_f16 per 16 dims for the two tiles. The
//     k slots 8j..8j+7 of lane (n, j) are tokens 4j..4j+3 of the first tile,
//     then of the second: the scores the lane already holds, so P goes from
//     the score MFMA to the value MFMA without leaving the lane. P enters in
//     fp16, pre-scaled by its tile's V scale and 2^-ve (ve from the wave's
//     largest V scale, so that p * scale_V * 2^-ve <= 2^15 with p <= 2^8);
//     the V codes, biased like K, are staged in LDS row-major and read
//     transposed with ds_read_b64_tr_b8 (within a 16-lane group, output lane
//     i receives byte i % 8 of source lanes i / 8 + 2k, k = 0..7: checked on
//     gfx950 with a one-wave probe); the bias part 1152 * sum_t P[t] is kept
//     in vb and removed at the end.
// Masked tokens (past the context, or of a tile whose id is out of range)
// get probability 0; their codes are finite, so they add exact zeros. The
// wave's (m, l, o[D]) per head go to mo ([G][D]) and mml ([G][2]).
template <int D, int G>
__device__ __forceinline__ void wave_stream_i8(const DecodeParams& prm, int g, int blk_lane, int n_my, int first,
                                               int ctx, const half8_t (&qa)[D / 32], float* mo, float* mml) {
  constexpr int NCH = D / 32;   // score MFMA chunks of 32 dims
  constexpr int NDB = D / 16;   // value MFMA blocks of 16 dims
  constexpr int KL = D / 64;    // K 16-byte loads per lane per tile
  constexpr int VL = D / 64;    // V 16-byte loads per lane per tile
  constexpr int VPR = D / 16;   // 16-byte pieces per V row
  constexpr int VR = D + 16;    // bytes per staged V row: the 16 rows of a tile on distinct bank offsets
  constexpr int TILE = BT * D;  // bytes per (block, KV head) tile
  __shared__ __align__(16) char vst_all[WAVES][2 * BT * VR];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 15, lj = lane >> 4;
  char* vst = vst_all[wave];
  const int Hkv = prm.Hkv;
  const char* Kc = static_cast<const char*>(prm.K);
  const char* Vc = static_cast<const char*>(prm.V);
  const int64_t head_off = int64_t(g) * TILE;
  const int64_t blk_stride = int64_t(Hkv) * TILE;

  // each tile's (K, V) scales, one pair per lane like the block ids; a tile
  // takes its pair with readlane when it is consumed
  const uint32_t sc_lane = unsigned(blk_lane) < unsigned(prm.num_blocks)
                               ? reinterpret_cast<const uint32_t*>(prm.scales)[int64_t(blk_lane) * Hkv + g]
                               : 0u;
  // 1152 * sum_d q[h][d] for this lane's head h = ln % G
  float qs = 0.0f;
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) qs += float(qa[c][e]);
  qs += xor_shfl(qs, 16);
  qs += xor_shfl(qs, 32);
  const float kbias = I8_BIAS * qs;

  float4_t ob[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) ob[i] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m = -INFINITY, l = 0.0f, vb = 0.0f;
  float vexp_scale = 1.0f, vexp_unscale = 1.0f;

  struct Pair {
    uint4 k[2][KL];
    uint4 v[2][VL];
    int blk[2];
  };
  // Tiles 2 pi and 2 pi + 1 (the second past n_my when n_my is odd: a
  // padding tile, loaded from block 0 and fully masked). it <= 63 always.
  auto load_pair = [&](int pi, Pair& t) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int blk = __builtin_amdgcn_readlane(blk_lane, 2 * pi + sub);
      t.blk[sub] = blk;
      const int safe = unsigned(blk) < unsigned(prm.num_blocks) ? blk : 0;
      const char* kb = Kc + safe * blk_stride + head_off;
      const char* vb_ = Vc + safe * blk_stride + head_off;
#pragma unroll
      for (int i = 0; i < KL; ++i) t.k[sub][i] = load_nt(kb + ln * D + (4 * i + lj) * 16);
#pragma unroll
      for (int i = 0; i < VL; ++i) {
        const int q = lane + 64 * i;
        t.v[sub][i] = load_nt(vb_ + (q / VPR) * D + (q % VPR) * 16);
      }
    }
  };

  // source address of this lane for the transpose read of dims 16 nb..: the
  // 16 lanes of group lj cover tokens 4 lj..4 lj + 3 of both tiles, two
  // 8-byte halves of the 16 dims each
  const int tr_ofs = ((ln >> 3) * BT + 4 * lj + ((ln >> 1) & 3)) * VR + 8 * (ln & 1);
  const half2_t ones = {(_Float16)1.0f, (_Float16)1.0f};

  auto compute_pair = [&](int pi, Pair& t) {
    // stage both V tiles (rows of D codes, padded)
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int i = 0; i < VL; ++i) {
        const int q = lane + 64 * i;
        *reinterpret_cast<uint4*>(vst + (sub * BT + q / VPR) * VR + (q % VPR) * 16) = t.v[sub][i];
      }
    float4_t acc[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      acc[sub] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint4& w = t.k[sub][c >> 1];
        uint32_t a0, a1, a2, a3;
        i8x4_to_f16x4_biased((c & 1) ? w.z : w.x, a0, a1);
        i8x4_to_f16x4_biased((c & 1) ? w.w : w.y, a2, a3);
        const half8_t kb = __builtin_bit_cast(half8_t, make_uint4(a0, a1, a2, a3));
        acc[sub] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kb, qa[c], acc[sub], 0, 0, 0);
      }
    }
    float s[8], vsc[2];
    bool ok[8];
    float smax = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int it = 2 * pi + sub;
      const uint32_t sc = __builtin_amdgcn_readlane(sc_lane, it);
      const float ks = prm.scale_log2 * lo_half(sc);
      const float kbs = kbias * ks;
      vsc[sub] = hi_half(sc) * vexp_scale;
      const int j = first + WAVES * it;
      const bool tile_ok = it < n_my && unsigned(t.blk[sub]) < unsigned(prm.num_blocks);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = 4 * sub + e;
        ok[k] = tile_ok && j * BT + 4 * lj + e < ctx;
        s[k] = ok[k] ? __builtin_fmaf(acc[sub][e], ks, -kbs) : -INFINITY;
        smax = fmaxf(smax, s[k]);
      }
    }
    if (__builtin_amdgcn_ballot_w64(smax > m + LAZY_MAX)) {  // wave-uniform, rare after the first step
      float mx = smax;
      mx = fmaxf(mx, xor_shfl(mx, 16));
      mx = fmaxf(mx, xor_shfl(mx, 32));
      const float mn = fmaxf(m, mx);
      const float alpha = (m == -INFINITY) ? 0.0f : exp2_fast(m - mn);
      m = mn;
      l *= alpha;
      vb *= alpha;
#pragma unroll
      for (int i = 0; i < NDB; ++i) ob[i] *= alpha;
    }
    half8_t pt;
#pragma unroll
    for (int k = 0; k < 8; k += 2) {
      const float p0 = ok[k] ? exp2_fast(s[k] - m) : 0.0f;
      const float p1 = ok[k + 1] ? exp2_fast(s[k + 1] - m) : 0.0f;
      l += p0 + p1;
      const half2_t ph = {(_Float16)(p0 * vsc[k >> 2]), (_Float16)(p1 * vsc[k >> 2])};
      vb = __builtin_amdgcn_fdot2(ph, ones, vb, false);
      pt[k] = ph.x;
      pt[k + 1] = ph.y;
    }
    // the staged V rows of the whole wave are visible to the transpose reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int nb = 0; nb < NDB; ++nb) {
      typedef int int2_t __attribute__((ext_vector_type(2)));
      const int2_t r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (__attribute__((address_space(3))) int2_t*)(vst + tr_ofs + 16 * nb));
      uint32_t a0, a1, b0, b1;
      i8x4_to_f16x4_biased(uint32_t(r.x), a0, a1);  // first tile, tokens 4j..4j+3
      i8x4_to_f16x4_biased(uint32_t(r.y), b0, b1);  // second tile
      const half8_t va = __builtin_bit_cast(half8_t, make_uint4(a0, a1, b0, b1));
      ob[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pt, ob[nb], 0, 0, 0);
    }
    // the next step's stores stay behind these reads
    __builtin_amdgcn_wave_barrier();
  };

  auto take_vexp = [&]() {
    float vmax = fabsf(hi_half(sc_lane));
#pragma unroll
    for (int mk = 1; mk < 64; mk <<= 1) vmax = fmaxf(vmax, xor_shfl(vmax, mk));
    const int ve = vmax > 128.0f ? int(ceilf(__builtin_log2f(vmax))) - 7 : 0;
    vexp_scale = __builtin_ldexpf(1.0f, -ve);
    vexp_unscale = __builtin_ldexpf(1.0f, ve);
  };

  // Double-buffered over pairs: the next pair's loads are issued before the
  // current pair is used.
  const int npairs = (n_my + 1) / 2;
  if (npairs > 0) {
    Pair pa, pb;
    int pi = 0;
    load_pair(0, pa);
    take_vexp();
    for (; pi + 2 < npairs; pi += 2) {
      load_pair(pi + 1, pb);
      compute_pair(pi, pa);
      load_pair(pi + 2, pa);
      compute_pair(pi + 1, pb);
    }
    if (pi + 1 < npairs) {
      load_pair(pi + 1, pb);
      compute_pair(pi, pa);
      compute_pair(pi + 1, pb);
    } else {
      compute_pair(pi, pa);
    }
  }

  // row totals over the four token groups; rows n and n + G (...) hold the
  // same head, rows below G are written
  l += xor_shfl(l, 16);
  l += xor_shfl(l, 32);
  vb += xor_shfl(vb, 16);
  vb += xor_shfl(vb, 32);
  if (ln < G) {
    const float bias = I8_BIAS * vb;
#pragma unroll
    for (int nb = 0; nb < NDB; ++nb)
#pragma unroll
      for (int e = 0; e < 4; ++e) mo[ln * D + 16 * nb + 4 * lj + e] = (ob[nb][e] - bias) * vexp_unscale;
    if (lj == 0) {
      mml[2 * ln] = m;
      mml[2 * ln + 1] = l;
    }
  }
}

// The early loads of a segment starting at logical block jb of sequence b:
// this wave's block ids (lane it: block jb + wave + 4 it; the table row is
// max_blocks wide and padded, ids past the context are masked later) and q
// of the lane's head kn % G as the score MFMA operand (group kj's dims).
template <int D, int G, bool I8>
__device__ __forceinline__ void segment_loads(const DecodeParams& prm, int g, int b, int jb, int& blk_raw,
                                              half8_t (&qa)[D / 32]) {
  using S = Shape<D, G, I8>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kn = lane & 15, kj = lane >> 4;
  const int jl = jb + wave + WAVES * lane;
  blk_raw = jl < prm.max_blocks ? prm.tables[int64_t(b) * prm.max_blocks + jl] : -1;
  const int gr = prm.group, h = kn % G;  // heads gr .. G - 1 of the kernel's group are padding (zero q)
  const _Float16* qh = prm.q + (int64_t(b) * prm.Hkv * gr + g * gr + min(h, gr - 1)) * D;
#pragma unroll
  for (int c = 0; c < S::NCH; ++c) {
    const u32x4 w = h < gr ? *reinterpret_cast<const u32x4*>(qh + S::dim_base(c, kj)) : u32x4{0u, 0u, 0u, 0u};
    qa[c] = __builtin_bit_cast(half8_t, w);
  }
}

// One segment of a decode work-group: logical blocks jb .. je - 1 of
// sequence b (context ctx) for KV head g. Wave w takes blocks jb + w,
// jb + w + 4, ...: its it-th id sits in lane it of blk_raw (loaded by
// segment_loads, with qa, before the context length is known, so a
// work-group waits one memory round trip before its first tile), and each
// tile reads it with readlane, so the id never waits on the vector memory
// queue. The 4 waves' results merge in LDS in fixed order; the work-group
// writes the final fp16 rows (final_row) or one (m, l, o[D]) partial per
// query head into slot `slot` of the head's partial row. append_here: the
// segment holds the sequence's last block, where the fused append writes
// the new token. Every thread of the work-group must call it.
template <int D, int G, bool I8>
__device__ __forceinline__ void decode_segment(const DecodeParams& prm, int g, int b, int ctx, int jb, int je,
                                               bool append_here, bool final_row, int slot, int blk_raw,
                                               const half8_t (&qa)[D / 32], float (&p_lds)[WAVES][BT][G],
                                               float (&merge_o)[WAVES][G][D], float (&merge_ml)[WAVES][G][2]) {
  using S = Shape<D, G, I8>;
  const int Hkv = prm.Hkv, gr = prm.group, Hq = Hkv * gr;  // heads gr .. G - 1 are padding
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int kn = lane & 15, kj = lane >> 4;  // score mapping: token, k-slot group
  const int vt = lane / S::LPR, vd = lane % S::LPR;  // V mapping: row group, dims
  const bool odd = (kj & 1) != 0;  // G == 8: this lane's score rows are heads 4..7

  const int32_t* trow = prm.tables + int64_t(b) * prm.max_blocks;
  const int first = jb + wave;
  const int n_my = first < je ? (je - first + WAVES - 1) / WAVES : 0;  // <= 64
  const int blk_lane = lane < n_my ? blk_raw : -1;

  const char* Kc = static_cast<const char*>(prm.K);
  const char* Vc = static_cast<const char*>(prm.V);
  const int64_t head_off = int64_t(g) * S::TILE;
  const int64_t blk_stride = int64_t(Hkv) * S::TILE;

  // Fused append: the new token is the last of the context, at logical
  // position ctx - 1, in this sequence's last segment. That work-group
  // writes its k and v rows for head g into the slot the table gives (fp16:
  // a bitwise copy; int8: quantised on write, its block's scale raised and
  // earlier rows re-rounded when needed), then reads them back with the rest
  // of the tile; no other work-group reads that block of this head in the
  // launch (a slot written at a non-zero offset of a shared block was moved
  // to a private block by copy-on-write).
  if (prm.k_new && append_here) {
    const int t = ctx - 1;
    const int blk = trow[t / BT];
    if (unsigned(blk) < unsigned(prm.num_blocks)) {
      if constexpr (I8) {
        if (wave < 2) {  // wave 0 writes the K row, wave 1 the V row
          const _Float16* src = reinterpret_cast<const _Float16*>(wave ? prm.v_new : prm.k_new) +
                                (int64_t(b) * Hkv + g) * D;
          int8_t* tile = reinterpret_cast<int8_t*>(const_cast<char*>(wave ? Vc : Kc) + blk * blk_stride + head_off);
          _Float16* sp = const_cast<_Float16*>(prm.scales) + (int64_t(blk) * Hkv + g) * 2 + wave;
          float x[D / 64];
#pragma unroll
          for (int e = 0; e < D / 64; ++e) x[e] = float(src[lane + 64 * e]);
          const float sn = quantise_row_i8<D>(tile, t % BT, x, float(*sp));
          if (lane == 0) *sp = _Float16(sn);
        }
      } else {
        constexpr int PIECES = D / 8;  // 16-byte pieces per fp16 row
        if (tid < 2 * PIECES) {
          const int c = tid % PIECES;
          const uint4* src = (tid < PIECES ? prm.k_new : prm.v_new) + (int64_t(b) * Hkv + g) * PIECES + c;
          char* dst = const_cast<char*>(tid < PIECES ? Kc : Vc) + blk * blk_stride + head_off + (t % BT) * (D * 2);
          reinterpret_cast<uint4*>(dst)[c] = *src;
        }
      }
      __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();
  }

  if constexpr (I8) {
    wave_stream_i8<D, G>(prm, g, blk_lane, n_my, first, ctx, qa, &merge_o[wave][0][0], &merge_ml[wave][0][0]);
  } else {
  // mh: running max per head (wave-uniform); lrow: this lane's share of the
  // softmax denominator per score row; o: V accumulators, D/16 dims x G heads
  float mh[G], o[G][S::CE], lrow[4];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    mh[h] = -INFINITY;
#pragma unroll
    for (int e = 0; e < S::CE; ++e) o[h][e] = 0.0f;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) lrow[e] = 0.0f;

  struct Tile {
    uint4 k[S::KL];
    uint4 v[S::NI];
    int blk;
  };

  // A bad id (outside the pool) still loads block 0, which exists; compute()
  // then masks every row of that tile.
  auto load = [&](int it, Tile& t) {
    const int blk = __builtin_amdgcn_readlane(blk_lane, it);
    t.blk = blk;
    const int safe = unsigned(blk) < unsigned(prm.num_blocks) ? blk : 0;
    const char* kb = Kc + safe * blk_stride + head_off;
    const char* vb = Vc + safe * blk_stride + head_off;
#pragma unroll
    for (int i = 0; i < S::KL; ++i) t.k[i] = load_nt(kb + kn * (D * S::E) + (4 * i + kj) * 16);
#pragma unroll
    for (int i = 0; i < S::NI; ++i) t.v[i] = load_nt(vb + (vt + S::RPI * i) * (D * S::E) + vd * 16);
  };

  // running max of the head of each of this lane's 4 score rows
  auto mrows = [&]() -> float4_t {
    if constexpr (G == 8) {
      return half_of8(mh, odd);
    } else {
      float4_t r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = mh[e % G];
      return r;
    }
  };

  auto compute = [&](int j, Tile& t) {
    const bool blk_ok = unsigned(t.blk) < unsigned(prm.num_blocks);
    const float kscale = prm.scale_log2;
    float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < S::NCH; ++c)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[c], __builtin_bit_cast(half8_t, t.k[c]), acc, 0, 0, 0);
    // A score of a row past the context (stale or poisoned) only reaches its
    // own column, and is replaced by -inf here.
    const bool tvalid = blk_ok && (j * BT + kn) < ctx;
    float s[4];
    bool need = false;
    float4_t mr = mrows();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s[e] = tvalid ? acc[e] * kscale : -INFINITY;
      need |= s[e] > mr[e] + LAZY_MAX;
    }
    if (__builtin_amdgcn_ballot_w64(need)) {  // wave-uniform, rare after the first tile
      float mx[G];
#pragma unroll
      for (int e = 0; e < 4 && e < G; ++e) {
        const float r = row16_max(s[e]);
        mx[e] = read_lane(r, 0);
        if constexpr (G == 8) mx[4 + e] = read_lane(r, 16);
      }
      float alpha[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mn = fmaxf(mh[h], mx[h]);
        alpha[h] = (mh[h] == -INFINITY) ? 0.0f : exp2_fast(mh[h] - mn);
        mh[h] = mn;
#pragma unroll
        for (int e = 0; e < S::CE; ++e) o[h][e] *= alpha[h];
      }
      if constexpr (G == 8) {
        const float4_t a4 = half_of8(alpha, odd);
#pragma unroll
        for (int e = 0; e < 4; ++e) lrow[e] *= a4[e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) lrow[e] *= alpha[e % G];
      }
      mr = mrows();
    }
    float pr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pr[e] = tvalid ? exp2_fast(s[e] - mr[e]) : 0.0f;
      lrow[e] += pr[e];
    }
    // hand the probabilities to the V lane mapping through LDS
    if constexpr (G == 8) {
      if (lane < 32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) p_lds[wave][kn][4 * kj + e] = pr[e];
      }
    } else {
      if (lane < 16) {
#pragma unroll
        for (int e = 0; e < G && e < 4; ++e) p_lds[wave][kn][e] = pr[e];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float pv[S::NI][G];
#pragma unroll
    for (int i = 0; i < S::NI; ++i)
#pragma unroll
      for (int h = 0; h < G; ++h) pv[i][h] = p_lds[wave][vt + S::RPI * i][h];
    // rows past the context (stale or poisoned) must contribute exact zeros
    const bool tail = !blk_ok || (j + 1) * BT > ctx;
    if (tail) {
#pragma unroll
      for (int i = 0; i < S::NI; ++i)
        if (!blk_ok || j * BT + vt + S::RPI * i >= ctx) t.v[i] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < S::NI; ++i) {
      const uint32_t w4[4] = {t.v[i].x, t.v[i].y, t.v[i].z, t.v[i].w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          o[h][2 * w + 0] = fmaf(pv[i][h], lo_half(w4[w]), o[h][2 * w + 0]);
          o[h][2 * w + 1] = fmaf(pv[i][h], hi_half(w4[w]), o[h][2 * w + 1]);
        }
      }
    }
    // the next tile rewrites p_lds: its writes stay behind these reads
    __builtin_amdgcn_wave_barrier();
  };

  // Double-buffered stream over this wave's tiles: in the steady state the
  // next tile's loads are always issued before the current tile is used, so
  // the wait before compute covers only the older tile.
  if (n_my > 0) {
    Tile ta, tb;
    int it = 0;
    load(0, ta);
    for (; it + 2 < n_my; it += 2) {
      load(it + 1, tb);
      compute(first + WAVES * it, ta);
      load(it + 2, ta);
      compute(first + WAVES * (it + 1), tb);
    }
    if constexpr (G == 8) {
      // one copy of each half of the tail (a uniform branch around the
      // second): the three-copy tail below would need more than 256 VGPRs
      // at eight heads
      const bool two = it + 1 < n_my;
      if (two) load(it + 1, tb);
      compute(first + WAVES * it, ta);
      if (two) compute(first + WAVES * (it + 1), tb);
    } else if (it + 1 < n_my) {
      load(it + 1, tb);
      compute(first + WAVES * it, ta);
      compute(first + WAVES * (it + 1), tb);
    } else {
      compute(first + WAVES * it, ta);
    }
  }

  // wave totals: l over the 16 tokens of each score row, o over the V row groups
  float lh[G];
#pragma unroll
  for (int e = 0; e < 4 && e < G; ++e) {
    const float r = row16_sum(lrow[e]);
    lh[e] = read_lane(r, 0);
    if constexpr (G == 8) lh[4 + e] = read_lane(r, 16);
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < S::CE; ++e)
#pragma unroll
      for (int mask = S::LPR; mask < 64; mask <<= 1) o[h][e] += xor_shfl(o[h][e], mask);
  if (vt == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < S::CE; ++e) merge_o[wave][h][vd * S::CE + e] = o[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      merge_ml[wave][h][0] = mh[h];
      merge_ml[wave][h][1] = lh[h];
    }
  }
  }  // fp16 stream
  __syncthreads();

  // merge the 4 waves (fixed order); write the final row or this partition's partial
  for (int idx = tid; idx < gr * D; idx += 256) {
    const int h = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) M = fmaxf(M, merge_ml[w][h][0]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const float mw = merge_ml[w][h][0];
      const float wt = (mw == -INFINITY) ? 0.0f : exp2_fast(mw - M);
      L += merge_ml[w][h][1] * wt;
      O += merge_o[w][h][d] * wt;
    }
    const int64_t row = int64_t(b) * Hq + g * gr + h;
    if (final_row) {
      prm.out[row * D + d] = (_Float16)(L > 0.0f ? O / L : 0.0f);
    } else {
      const int64_t pi = row * prm.max_parts + slot;
      prm.part_o[pi * D + d] = O;
      if (d == 0) {
        prm.part_m[pi] = M;
        prm.part_l[pi] = L;
      }
    }
  }
}

// Stream-K split (ragged batches with host lengths, no plan). The blocks of
// all sequences, laid end to end (sequence 0's, then 1's, ...), each span
// led by prm.stream_pad blocks that stand for the start-up of a piece and
// hold no work, are cut into runs of q = prm.part_blocks blocks, one per
// work-group of a KV head: work-group k covers [k q, (k + 1) q), which may
// end one sequence and start the next (and then holds fewer real blocks).
// Each piece of a sequence it covers is a segment with its own partial, in
// slot k - floor(C_b / q) of the sequence's partial rows (C_b: the
// sequence's first real block in the run); a sequence that one work-group
// covers entirely gets its final rows from it. Every sequence's C_b comes
// from a work-group-wide scan of all lengths. Sequences
// without tokens are skipped (the host rejects them when it has the lengths).
// With a shared-prefix plan a grouped sequence's span starts after its
// shared blocks, and its partials follow the group's prefix partials.
template <int D, int G, bool I8, bool PLAN>
__device__ __forceinline__ void stream_k_role(const DecodeParams& prm, int g, int k, float (&p_lds)[WAVES][BT][G],
                                              float (&merge_o)[WAVES][G][D], float (&merge_ml)[WAVES][G][2]) {
  __shared__ int seq_first[STREAM_MAX_SEQS + 1];
  __shared__ int seq_ctx[STREAM_MAX_SEQS];
  static_assert(sizeof(merge_o) >= WAVES * sizeof(int), "scan scratch");
  int* part = reinterpret_cast<int*>(&merge_o[0][0][0]);
  const int tid = threadIdx.x;
  const int B = prm.num_seqs, q = prm.part_blocks;
  constexpr int PER = STREAM_MAX_SEQS / 256;
  int n[PER], c[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {  // all lengths in flight together
    const int t = tid + 256 * i;
    c[i] = t < B ? clamp_ctx(prm.ctx_lens[t], prm.max_blocks, prm.max_context) : 0;
    int sb = 0, pre;
    if (PLAN && t < B) seq_prefix(prm.plan, t, prm.max_blocks, prm.num_groups, prm.prefix_pp, sb, pre);
    n[i] = c[i] > 0 ? max((c[i] + BT - 1) / BT - sb, 0) : 0;  // the span after the shared blocks
    n[i] += n[i] > 0 ? prm.stream_pad : 0;                   // and its start-up charge ahead of it
  }
  int carry = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (256 * i >= B) break;  // uniform
    int tot;
    const int ex = carry + wg_exclusive_scan(n[i], part, tot);
    const int t = tid + 256 * i;
    if (t < B) {
      seq_first[t] = ex;
      seq_ctx[t] = c[i];
    }
    carry += tot;
  }
  if (tid == 0) seq_first[B] = carry;
  __syncthreads();
  const int T = seq_first[B];
  const int lo = k * q;
  if (lo >= T) return;  // uniform
  const int hi = min(lo + q, T);
  int b = 0, r = B;  // the last sequence whose first block is at or before lo
  while (r - b > 1) {
    const int m = (b + r) / 2;
    if (seq_first[m] <= lo) b = m;
    else r = m;
  }
  for (;;) {
    // sequence b's real blocks: [cb, cn), after its start-up charge
    const int cn = seq_first[b + 1], cb = min(seq_first[b] + prm.stream_pad, cn);
    if (cn > cb && hi > cb) {
      int sb = 0, pre = 0;  // a grouped sequence's span starts after its shared blocks; its prefix partials first
      if constexpr (PLAN) seq_prefix(prm.plan, b, prm.max_blocks, prm.num_groups, prm.prefix_pp, sb, pre);
      const int s0 = max(lo, cb) - cb, s1 = min(hi, cn) - cb;
      const int first_wg = cb / q, count = (cn - 1) / q - first_wg + 1;
      int blk_raw;
      half8_t qa[D / 32];
      segment_loads<D, G, I8>(prm, g, b, sb + s0, blk_raw, qa);
      decode_segment<D, G, I8>(prm, g, b, seq_ctx[b], sb + s0, sb + s1, s1 == cn - cb, count == 1 && pre == 0,
                               pre + k - first_wg, blk_raw, qa, p_lds, merge_o, merge_ml);
      __syncthreads();  // the next segment reuses the wave-merge buffers
    }
    if (cn >= hi || ++b >= B) break;
  }
}

// Two work-groups per CU are asked of the register allocator where they
// fit without spills (G <= 4; fp16 at D = 64): the shared-prefix role would
// otherwise push the fp16 kernels past 256 registers a lane. The other
// G = 8 kernels keep the full register file.
//
// One work-group (4 wave64s) per (KV head g, sequence b, partition p), in
// that grid order (x, y, z). Work-groups go to the eight XCDs round-robin by
// linear id, so the partition index, the dimension along which work runs out
// first (short sequences, or a shared prefix attended elsewhere), varies
// slowest: the busy work-groups of any one partition index are spread over
// all XCDs instead of piling onto those whose id matches a low index.
//
// Scores on the matrix cores: per tile, S[r][n] = sum_k Q[r][k] K[n][k] with
// v_mfma_f32_16x16x32_f16 over D/32 chunks. A-row r holds query head r % G of
// the group (rows repeat when G < 16), B-column n is token n of the tile.
// Lane (n = lane % 16, j = lane / 16) feeds token n's K dims of k-slot group
// j and receives rows 4j..4j+3 of column n: the scores of heads
// (4j + e) % G, e = 0..3, for its token, already fully reduced.
//
// After its last tile the work-group writes one (m, l, o[D]) partial per
// query head for the merge kernel, or the final fp16 row when the sequence
// has a single partition.
// GRID_STREAM: the stream-K split above, chosen by the host from its copy
// of the lengths for ragged batches. The plain grid holds max-context
// partitions for every sequence, and a work-group past its sequence's last
// partition exits once its length has arrived; under a full HBM stream that
// holds its slot for microseconds, and real work-groups queue behind such
// exits. GRID_PLAN: the plain grid led by the shared-prefix planes; the
// multi-row attention of that role needs more registers than the split
// role, so launches without a plan use GRID_PLAIN, which leaves it out.
enum { GRID_PLAIN = 0, GRID_STREAM = 1, GRID_PLAN = 2 };

// Work-groups per CU the decode kernels are built for (two waves per SIMD,
// at most 256 VGPRs, or one). fp16 at eight query heads per KV head holds
// twice the value accumulators; with its stream's tail written once per
// half it fits 256 VGPRs (219 on the plain grid, 234 plan), and two per CU
// beat one: 16 x 8193 tokens, 64 q / 8 KV heads, 88.3-88.5 us against
// 91.0-91.3; the shared-prefix launch over 32 members of a 2048-token
// prefix at 64 q / 8 KV heads, 27.5-27.7 us against 40.4-40.7. Its
// stream-K grid measured no faster at two and is built for one (241 VGPRs)
// and held there by the host (see cap_per_cu_lds).
template <bool I8, int D, int G, int GRID>
constexpr int decode_wgs_per_cu() {
  return (I8 || G <= 4 || GRID != GRID_STREAM) ? 2 : 1;
}

template <int D, int G, bool I8, int GRID>
__global__ __launch_bounds__(256, (decode_wgs_per_cu<I8, D, G, GRID>())) void paged_decode_kernel(DecodeParams prm) {
  const int g = blockIdx.x;
  __shared__ float p_lds[WAVES][BT][G];
  __shared__ float merge_o[WAVES][G][D];
  __shared__ float merge_ml[WAVES][G][2];
  if constexpr (GRID == GRID_STREAM) {
    stream_k_role<D, G, I8, false>(prm, g, blockIdx.y + gridDim.y * blockIdx.z, p_lds, merge_o, merge_ml);
    return;
  } else if constexpr (GRID == GRID_PLAN) {
    // With a shared-prefix plan the grid leads with the shared-prefix
    // work-groups: dispatched first, they run beside the split work-groups of
    // the same launch, which follow them (stream-K, when the host has both
    // the lengths and the plan) or fill the planes after the first prefix_z.
    const int k = blockIdx.y + gridDim.y * blockIdx.z;
    const int units = prm.prefix_pp * prm.num_groups * PREFIX_SPLIT;
    if (prm.plan_stream ? k < units : int(blockIdx.z) < prm.prefix_z) {
      const int unit = k / PREFIX_SPLIT;
      if (unit < prm.prefix_pp * prm.num_groups)
        prefix_role<D, G, I8>(prm, g, unit / prm.prefix_pp, unit % prm.prefix_pp, k % PREFIX_SPLIT);
      return;
    }
    if (prm.plan_stream) {
      stream_k_role<D, G, I8, true>(prm, g, k - units, p_lds, merge_o, merge_ml);
      return;
    }
  }
  const int b = blockIdx.y;
  const int p = int(blockIdx.z) - (GRID == GRID_PLAN ? prm.prefix_z : 0);
  // With a shared-prefix plan, a grouped sequence's leading shared blocks are
  // attended by the shared-prefix work-groups: partitions start after them,
  // and their partials follow the `pre` prefix partials in the partial row.
  int sb, pre;
  seq_prefix(prm.plan, b, prm.max_blocks, prm.num_groups, prm.prefix_pp, sb, pre);
  const int jb = sb + p * prm.part_blocks;
  // the block ids and q are loaded with the context length: one round trip
  int blk_raw;
  half8_t qa[D / 32];
  segment_loads<D, G, I8>(prm, g, b, jb, blk_raw, qa);
  const int ctx = clamp_ctx(prm.ctx_lens[b], prm.max_blocks, prm.max_context);
  if (ctx <= 0) {  // rejected on the host when lengths are given; never NaN
    if (p == 0)
      for (int i = threadIdx.x; i < prm.group * D; i += 256)
        prm.out[(int64_t(b) * prm.Hkv * prm.group + g * prm.group) * D + i] = _Float16(0.0f);
    return;
  }
  const int nblk = (ctx + BT - 1) / BT;
  const int nparts = nblk > sb ? (nblk - sb + prm.part_blocks - 1) / prm.part_blocks : 0;
  if (p >= nparts) return;
  decode_segment<D, G, I8>(prm, g, b, ctx, jb, min(nblk, jb + prm.part_blocks), p == nparts - 1,
                           nparts == 1 && pre == 0, pre + p, blk_raw, qa, p_lds, merge_o, merge_ml);
}

struct MergeParams {
  const float* part_m;  // partials [B][Hq][max_parts] (+ [D]): prefix, then split-K
  const float* part_l;
  const float* part_o;
  const int32_t* ctx_lens;
  const int32_t* plan;  // null = no shared-prefix plan
  _Float16* out;
  int D, max_blocks, max_context, part_blocks, max_parts;
  int num_groups, prefix_pp;
  int row_parts;  // partials any row of this launch can hold (<= max_parts)
  int num_seqs;
  int stream_q;   // stream-K split: blocks per work-group (0 = partitions of part_blocks per sequence)
  int stream_pad;  // stream-K split: start-up charge ahead of each span (as in DecodeParams)
};

// Stream-K split: the blocks sequence b's span (its blocks after any shared
// ones) has and where it starts in the run of all spans, summed over the
// work-group's threads (tid of nthreads, at most 1024), every thread
// receiving it. red: 16 ints of LDS.
__device__ __forceinline__ int span_blocks(const MergeParams& prm, int t) {
  const int c = clamp_ctx(prm.ctx_lens[t], prm.max_blocks, prm.max_context);
  int sb, pre;
  seq_prefix(prm.plan, t, prm.max_blocks, prm.num_groups, prm.prefix_pp, sb, pre);
  return c > 0 ? max((c + BT - 1) / BT - sb, 0) : 0;
}
// the span's length in the run: its blocks and, when it has any, the
// start-up charge laid ahead of them
__device__ __forceinline__ int run_blocks(const MergeParams& prm, int t) {
  const int n = span_blocks(prm, t);
  return n > 0 ? n + prm.stream_pad : 0;
}
__device__ __forceinline__ int run_first_block(const MergeParams& prm, int b, int tid, int nthreads, int* red) {
  int sum = 0;
  for (int t = tid; t < b; t += nthreads) sum += run_blocks(prm, t);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) sum += __shfl_xor(sum, m, 64);
  const int wave = tid >> 6, waves = (nthreads + 63) >> 6;
  if ((tid & 63) == 0) red[wave] = sum;
  __syncthreads();
  int total = 0;
  for (int w = 0; w < waves; ++w) total += red[w];
  return total;
}

// Merge the partials of one (sequence, query head) by log-sum-exp:
// M = max_p m_p, out = sum_p o_p 2^(m_p - M) / sum_p l_p 2^(m_p - M), in
// logical order: the shared-prefix partials of the sequence's group (if it
// has one), then its own split-K partitions, which follow them in the
// sequence's partial row. A work-group of D x W threads (W = blockDim.y,
// the number of partial streams): thread (d, w) folds output dim d of
// partials w, w + W, ... (16 at a time, all loads of a group in flight
// together, the first group with the context length and the plan; across
// groups the running max is raised as in the split kernel), and with W > 1
// the W results are combined through LDS in order w = 0, 1, ... by the same
// formula. Several streams keep the chain of dependent loads short when
// rows have many partials (short sequences cut into many partitions); with
// few, one stream is cheaper. Sequences with a single partial were finished
// by the split kernel. The first group loads only slots below row_parts (the
// launch's prefix partitions + split planes): slots past it were not written
// by this launch.
constexpr int MERGE_MAX_WAYS = 8;
// Partial streams per merged row for launches whose rows hold up to
// max_parts partials (measured on MI355X: one stream up to 32 partials).
int merge_ways(int max_parts) { return max_parts <= 32 ? 1 : max_parts <= 128 ? 4 : MERGE_MAX_WAYS; }

__global__ __launch_bounds__(1024) void lse_reduce_kernel(MergeParams prm) {
  constexpr int CH = 16;
  const int h = blockIdx.x, b = blockIdx.y, Hq = gridDim.x;
  const int d = threadIdx.x, w = threadIdx.y, W = blockDim.y;  // blockDim = (D, W), D <= 128, W <= 8
  const int D = prm.D;
  __shared__ float part_mo[MERGE_MAX_WAYS][128];
  __shared__ float part_ml[MERGE_MAX_WAYS][2];
  const int64_t base = (int64_t(b) * Hq + h) * prm.max_parts;
  float m0[CH], l0[CH], o0[CH];
#pragma unroll
  for (int u = 0; u < CH; ++u) {
    const int p = w + W * u;
    if (p < prm.row_parts) {  // uniform over the launch
      const int64_t pi = base + p;
      m0[u] = prm.part_m[pi];
      l0[u] = prm.part_l[pi];
      o0[u] = prm.part_o[pi * D + d];
    } else {
      m0[u] = -INFINITY;
      l0[u] = 0.0f;
      o0[u] = 0.0f;
    }
  }
  int sb, pre;
  seq_prefix(prm.plan, b, prm.max_blocks, prm.num_groups, prm.prefix_pp, sb, pre);
  const int ctx = clamp_ctx(prm.ctx_lens[b], prm.max_blocks, prm.max_context);
  const int nblk = ctx > 0 ? (ctx + BT - 1) / BT : 0;
  int nparts;
  if (prm.stream_q > 0) {  // the stream-K work-groups that covered the sequence's span, in order
    __shared__ int red[16];
    const int cb = run_first_block(prm, b, d + D * w, D * W, red) + prm.stream_pad;  // first real block
    const int span = ctx > 0 ? max(nblk - sb, 0) : 0;
    nparts = span > 0 ? (cb + span - 1) / prm.stream_q - cb / prm.stream_q + 1 : 0;
  } else {
    nparts = nblk > sb ? (nblk - sb + prm.part_blocks - 1) / prm.part_blocks : 0;
  }
  if (ctx <= 0) return;  // uniform over the work-group
  if (pre == 0 && nparts <= 1) return;
  const int count = min(pre + nparts, prm.row_parts);

  float M = -INFINITY, L = 0.0f, O = 0.0f;
  for (int k0 = 0; w + W * k0 < count; k0 += CH) {
    float mv[CH], lv[CH], ov[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int p = w + W * (k0 + u);
      const bool ok = p < count;
      if (k0 == 0) {
        mv[u] = ok ? m0[u] : -INFINITY;
        lv[u] = ok ? l0[u] : 0.0f;
        ov[u] = ok ? o0[u] : 0.0f;
      } else {
        const int64_t pi = base + (ok ? p : 0);
        mv[u] = ok ? prm.part_m[pi] : -INFINITY;
        lv[u] = ok ? prm.part_l[pi] : 0.0f;
        ov[u] = ok ? prm.part_o[pi * D + d] : 0.0f;
      }
    }
    float cm = M;
#pragma unroll
    for (int u = 0; u < CH; ++u) cm = fmaxf(cm, mv[u]);
    if (cm != M) {  // raise the running max (always on the first group)
      const float a = (M == -INFINITY) ? 0.0f : exp2_fast(M - cm);
      L *= a;
      O *= a;
      M = cm;
    }
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const float wt = (mv[u] == -INFINITY) ? 0.0f : exp2_fast(mv[u] - M);
      L += lv[u] * wt;
      O += ov[u] * wt;
    }
  }
  const int64_t oi = (int64_t(b) * Hq + h) * D + d;
  if (W == 1) {  // uniform over the launch
    prm.out[oi] = (_Float16)(L > 0.0f ? O / L : 0.0f);
    return;
  }
  part_mo[w][d] = O;
  if (d == 0) {
    part_ml[w][0] = M;
    part_ml[w][1] = L;
  }
  __syncthreads();
  if (w != 0) return;
  float Mt = -INFINITY;
  for (int v = 0; v < W; ++v) Mt = fmaxf(Mt, part_ml[v][0]);
  float Lt = 0.0f, Ot = 0.0f;
  for (int v = 0; v < W; ++v) {
    const float mw = part_ml[v][0];
    const float wt = (mw == -INFINITY) ? 0.0f : exp2_fast(mw - Mt);
    Lt += part_ml[v][1] * wt;
    Ot += part_mo[v][d] * wt;
  }
  prm.out[oi] = (_Float16)(Lt > 0.0f ? Ot / Lt : 0.0f);
}

// Host -> device staging of small host metadata (block tables, lengths): one
// thread per 16 bytes reads the pinned host buffer through its device mapping
// and writes device memory; the last thread copies a ragged tail byte-wise.
__global__ __launch_bounds__(256) void upload_kernel(char* __restrict__ dst, const char* __restrict__ src,
                                                     int64_t bytes) {
  const int64_t n16 = bytes / 16;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
    reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(src)[i];
  if (blockIdx.x == 0 && threadIdx.x == 0)
    for (int64_t i = n16 * 16; i < bytes; ++i) dst[i] = src[i];
}

// Coalesced streaming read of a buffer, for an achievable-bandwidth
// reference: 8 independent non-temporal 16-byte loads per thread in flight,
// grid-stride over the buffer (a tail shorter than one 8 x 256 x 16-byte
// stripe is not read).
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ buf, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  constexpr int U = 8;
  uint32_t acc = 0;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x * U;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x * U + threadIdx.x; i + int64_t(blockDim.x) * (U - 1) < n16;
       i += stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = load_nt(buf + i + int64_t(blockDim.x) * u);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;  // keeps the loads; practically never taken
}

// ---------------------------------------------------------------------------
// host side

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PKV_OK;
  return pkv::fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Blocks per split-K partition: explicit, from PKV_PARTITION_TOKENS, or
// about want_wgs work-groups over B x Hkv (sequence, KV head) pairs at
// max_context. The workspace is sized for 2048 work-groups; a launch never
// cuts finer than the workspace (its grid and partial rows stay within it)
// and usually cuts coarser, see launch_part_blocks. Partitions keep at least 16 blocks (four tiles per
// wave): small launches cut finer spend their time starting work-groups (8
// sequences at 1025 tokens: 14.0 us at 64-token partitions, 10.0 at 256; a
// 16-sequence 8K batch on one KV head: 20.5 us at 80 tokens, 14.4 at 512).
// The partitions of the longest sequence are then made equal.
constexpr int MIN_PART_BLOCKS = 16;
// Stream-K split: blocks of work charged for starting a sequence's piece.
// A work-group that crosses into the next sequence pays that piece's
// start-up (its block ids and q, the first tiles' latency, and the wave
// merge and partial write of the piece before): charging it as blocks laid
// ahead of every span gives such work-groups fewer real blocks.
int stream_pad_blocks(int dtype) { return dtype == PKV_I8 ? STREAM_PAD_I8 : STREAM_PAD_F16; }

int choose_part_blocks(int Hkv, int B, int max_context, int partition_tokens, int64_t want_wgs) {
  if (partition_tokens == 0) {
    if (const char* env = std::getenv("PKV_PARTITION_TOKENS")) partition_tokens = std::atoi(env);
  }
  if (partition_tokens > 0) return std::min(partition_tokens, MAX_PARTITION_TOKENS) / BT;
  const int nblk = (max_context + BT - 1) / BT;
  const int64_t groups = int64_t(B) * Hkv;
  int64_t want_parts = (want_wgs + groups - 1) / groups;
  if (want_parts < 1) want_parts = 1;
  int pb = int((nblk + want_parts - 1) / want_parts);
  pb = std::min(std::max(pb, MIN_PART_BLOCKS), MAX_PARTITION_TOKENS / BT);
  const int parts = (nblk + pb - 1) / pb;
  pb = (nblk + parts - 1) / parts;
  return std::max(pb, WAVES);  // at least one block per wave
}

// Decode work-groups the current device holds at once (CUs x work-groups
// per CU at the kernel's register and LDS use) and its CU count, per device
// and kernel.
struct Residency {
  int slots, cus;
};
Residency resident_wgs(const void* fn, size_t dyn_lds) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, Residency> known;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(dev, fn);
  const auto it = known.find(key);
  if (it != known.end()) return it->second;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, dyn_lds) != hipSuccess || per_cu < 1)
    per_cu = 1;
  if (dev < 0 || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  (void)hipGetLastError();  // a failed query above must not be reported by the launch
  return known[key] = Residency{per_cu * cus, cus};
}

// Dynamic LDS (unused by the kernel) that holds a decode launch to `cap`
// work-groups per CU where registers and static LDS would allow more:
//   * int8, cap 2: the int8 stream is HBM-bound and runs faster with two
//     longer-lived work-groups per CU (measured on MI355X, int8 batch 16 x
//     8192 tokens, same box: 45.1-45.4 us at two per CU against 47.0-47.2 at
//     three, and 45.9-46.1 with the two-per-CU cut on CUs that could take a
//     third);
//   * fp16 at eight query heads per KV head on the stream-K grid, cap 1
//     (two per CU measured no faster: ragged 16 x U[128, 8193], 64 q / 8 KV
//     heads, 57.1-57.4 us at two against 56.8-57.1 at one).
// 0 where at most `cap` fit anyway. Per device and kernel.
size_t cap_per_cu_lds(const void* fn, int cap) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, size_t> known;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(dev, fn);
  const auto it = known.find(key);
  if (it != known.end()) return it->second;
  size_t extra = 0;
  int per_cu = 0, lds_cu = 0;
  hipFuncAttributes attr;
  if (dev >= 0 && hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, 0) == hipSuccess && per_cu > cap &&
      hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) == hipSuccess &&
      hipFuncGetAttributes(&attr, fn) == hipSuccess) {
    const size_t want = size_t(lds_cu) / (cap + 1) + 1024;  // work-group cap + 1 no longer fits
    if (want > attr.sharedSizeBytes) extra = want - attr.sharedSizeBytes;
  }
  (void)hipGetLastError();  // a failed query above must not be reported by the launch
  return known[key] = extra;
}

// The dynamic LDS of a decode launch of kernel fn (built for kg query heads
// per KV head, on `grid`).
size_t decode_dyn_lds(const void* fn, bool i8, int kg, int grid) {
  if (i8) return cap_per_cu_lds(fn, 2);
  return kg == 8 && grid == GRID_STREAM ? cap_per_cu_lds(fn, 1) : 0;
}

// Blocks per partition for one launch. Each partition is one work-group and
// the decode is HBM-bound, so the fewest rounds of resident work-groups win:
// among the partition counts of the longest span (its partitions equal, at
// most 256 blocks, at least 16 and at least pb_min) that need the fewest
// rounds of `slots` work-groups, take the finest, which spreads the bytes over
// the most work-groups. span(b) is the number of blocks the split role
// covers for sequence b. Measured on MI355X against the workspace's
// 2048-work-group cut: batch 16 x 8193 tokens 86.1 -> 84.0 us (4 partitions,
// one round), lengths U[128, 8193] 46.2 -> 39.7 us, the same in int8 37.3 ->
// 30.0 us, 64 q heads 120.6 -> 90.1 us (two rounds of one work-group per CU),
// 16 sequences on 4 / 2 / 1 KV heads 48.6 / 25.6 / 15.7 -> 44.3 / 24.4 /
// 14.8 us, 4 x 32K tokens 88.3 -> 83.9 us; 64 x 2049 and 64 x 300 tokens
// drop the merge kernel (one partition each).
// When that one-round cut puts two work-groups on some CUs, the finest cut
// with at most one work-group per CU is taken instead if its partitions are
// at most twice as long (the load of a doubled CU): a CU holding two
// work-groups of a small launch streams them no faster than one longer one,
// and a partly filled second layer is a tail (measured on MI355X, split us,
// one-round cut -> this rule: 8 x 1025 tokens 11.9 -> 9.7 (13 -> 17 blocks,
// 320 -> 256 work-groups), 4 x 2049 11.7 -> 9.5, 8 x 2049 15.7 -> 14.6, two
// KV heads x 16 x 8193 25.1 -> 24.4). Large launches have no such cut (the
// batch-16 8K step would need 257-block partitions), and a ragged batch's
// is usually far coarser (the continuous-batching mix: 245 blocks against
// 82), so both keep the one-round cut.
template <typename Span>
int launch_part_blocks(int Hkv, int B, Span span, Residency res, int pb_min) {
  const int slots = res.slots;
  int nmax = 0;
  for (int b = 0; b < B; ++b) nmax = std::max(nmax, span(b));
  if (nmax < 1) return std::max(pb_min, 1);
  const int max_pb = MAX_PARTITION_TOKENS / BT;
  auto wgs = [&](int pb) {
    int64_t n = 0;
    for (int b = 0; b < B; ++b) n += (span(b) + pb - 1) / pb;
    return n * Hkv;
  };
  const int p_lo = std::max(1, (nmax + max_pb - 1) / max_pb);
  const int p_hi = std::max(p_lo, (nmax + MIN_PART_BLOCKS - 1) / MIN_PART_BLOCKS);
  auto blocks = [&](int parts) { return (nmax + parts - 1) / parts; };
  if (blocks(p_lo) < pb_min) return pb_min;
  const int64_t rounds = (wgs(blocks(p_lo)) + slots - 1) / slots;
  int best = p_lo;
  // past 4 rounds of pairs alone, finer cuts only add work-groups
  if (int64_t(B) * Hkv < 4 * int64_t(slots)) {
    for (int parts = p_lo + 1; parts <= p_hi; ++parts) {
      const int pb = blocks(parts);
      if (pb < pb_min) break;
      if (pb == blocks(best)) continue;
      if (wgs(pb) <= rounds * slots) best = parts;
    }
  }
  const int pb_round = blocks(best);
  const int64_t w_round = wgs(pb_round);
  if (rounds == 1 && w_round > res.cus) {
    // the finest cut with at most one work-group per CU, if its partitions
    // are no longer than what the doubled CUs of the one-round cut carry
    // (a ragged batch's longest sequence can make them far longer)
    for (int parts = p_hi; parts >= p_lo; --parts) {  // finest first
      const int pb = blocks(parts);
      if (pb < pb_min) continue;
      if (wgs(pb) <= res.cus) return pb <= 2 * pb_round ? pb : pb_round;
    }
  }
  return pb_round;
}

int max_parts_for(int max_context, int part_blocks) {
  const int nblk = (max_context + BT - 1) / BT;
  return (nblk + part_blocks - 1) / part_blocks;
}

typedef void (*decode_fn)(DecodeParams);

// A group of G query heads runs on the kernel built for the next size up
// (3 on 4; 5, 6 and 7 on 8): its extra heads get zero q and are never
// written, so they cost arithmetic and no bytes.
template <int D, bool I8, int GRID>
decode_fn pick_g(int G) {
  switch (G) {
    case 1: return paged_decode_kernel<D, 1, I8, GRID>;
    case 2: return paged_decode_kernel<D, 2, I8, GRID>;
    case 3:
    case 4: return paged_decode_kernel<D, 4, I8, GRID>;
    case 5:
    case 6:
    case 7:
    case 8: return paged_decode_kernel<D, 8, I8, GRID>;
    default: return nullptr;
  }
}

template <int GRID>
decode_fn pick_dt(int D, int G, bool i8) {
  if (D == 128) return i8 ? pick_g<128, true, GRID>(G) : pick_g<128, false, GRID>(G);
  if (D == 64) return i8 ? pick_g<64, true, GRID>(G) : pick_g<64, false, GRID>(G);
  return nullptr;
}

decode_fn pick_kernel(int D, int G, bool i8, int grid) {
  return grid == GRID_STREAM ? pick_dt<GRID_STREAM>(D, G, i8)
         : grid == GRID_PLAN  ? pick_dt<GRID_PLAN>(D, G, i8)
                              : pick_dt<GRID_PLAIN>(D, G, i8);
}

// Split-K workspace: m [B][Hq][P], l [B][Hq][P], o [B][Hq][P][D] (fp32); none
// when every sequence fits one partition.
int64_t workspace_bytes_for(const pkv_config& c, int B, int Hq, int max_parts) {
  if (max_parts <= 1) return 0;
  return int64_t(B) * Hq * max_parts * (c.head_dim + 2) * int64_t(sizeof(float));
}

// Prefix partitions per group. A partition adds 128 partial rows of D + 2
// floats (66.5 KB at D = 128) against 8 KB of K/V per shared block, and its
// work-group walks its blocks one tile after another, so partitions are
// neither short (partial traffic) nor long (the chain outlasts the split
// work-groups beside it): about 128 shared-prefix work-groups over groups
// and KV heads, 16 to 64 blocks each (measured on MI355X: 32 sequences over
// a 2048-token prefix run best at 96 work-groups of 11 blocks, 64 over two
// 4096-token prefixes at 160 of 26).
constexpr int PREFIX_TARGET_WGS = 128;
// With the plan's host copy the launch knows each group's shared blocks and
// cuts the longest run into partitions of about this many blocks (at most
// as many as the workspace holds). Measured on MI355X with the rows split
// over two work-groups and the stream-K split side, 32 sequences over a
// 2048-token prefix (128 shared blocks): 4 partitions of 32 blocks 22.1 us
// per launch, 5 of 26 22.7, 7 of 19 24.4, 10 of 13 27.4, 2 of 64 30.1, one
// of 128 46.6; one 4096-token prefix and two 3000-token prefixes were best
// at 32 blocks as well.
constexpr int PREFIX_PART_BLOCKS = 32;
int prefix_partitions(int Hkv, int n_groups, int max_blocks) {
  const int64_t lo = (int64_t(max_blocks) + 63) / 64;  // <= 64 blocks: the block ids staged in LDS
  const int64_t hi = std::max<int64_t>(lo, (max_blocks + 15) / 16);
  const int64_t want = (PREFIX_TARGET_WGS + int64_t(Hkv) * n_groups - 1) / (int64_t(Hkv) * n_groups);
  return int(std::min(hi, std::max(lo, want)));
}

// Workspace of one decode: partial rows m [B][Hq][P], l [B][Hq][P],
// o [B][Hq][P][D] (fp32). Without a plan P is the split-K partition count
// (no workspace when it is 1). With a shared-prefix plan every row also
// holds up to prefix_pp prefix partials ahead of the split-K ones, and the
// grid gains prefix_z planes of shared-prefix work-groups (one per group,
// prefix partition and KV head).
struct WsLayout {
  int part_blocks, grid_parts, max_parts, prefix_pp, prefix_z;
  int64_t bytes;
};

WsLayout ws_layout(const pkv_config& c, int B, int Hq, int max_context, int max_blocks, int partition_tokens,
                   int n_groups) {
  WsLayout w;
  w.part_blocks = choose_part_blocks(c.num_kv_heads, B, max_context, partition_tokens, 2048);
  w.grid_parts = max_parts_for(max_context, w.part_blocks);
  w.prefix_pp = n_groups > 0 ? prefix_partitions(c.num_kv_heads, n_groups, max_blocks) : 0;
  w.prefix_z = n_groups > 0 ? int((int64_t(w.prefix_pp) * n_groups * PREFIX_SPLIT + B - 1) / B) : 0;
  w.max_parts = w.grid_parts + w.prefix_pp;
  w.bytes = n_groups > 0 ? int64_t(B) * Hq * w.max_parts * (c.head_dim + 2) * int64_t(sizeof(float))
                         : workspace_bytes_for(c, B, Hq, w.max_parts);
  return w;
}

int check_partition_tokens(int partition_tokens) {
  if (partition_tokens < 0 || partition_tokens % BT || partition_tokens > MAX_PARTITION_TOKENS)
    return pkv::fail(PKV_ERR_INVALID_ARG, "partition_tokens must be a multiple of 16 in [0, %d] (got %d)",
                     MAX_PARTITION_TOKENS, partition_tokens);
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_copy_blocks(const pkv_config* cfg, void* pool_dev, const int32_t* pairs_dev, int32_t n, void* stream) {
  int st = pkv::validate_config(cfg);
  if (st != PKV_OK) return st;
  if (n < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "n must be >= 0");
  if (n == 0) return PKV_OK;
  if (!pool_dev || !pairs_dev) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL device pointer");
  if (!aligned16(pool_dev)) return pkv::fail(PKV_ERR_INVALID_ARG, "pool must be 16-byte aligned");
  if (n > 65535) return pkv::fail(PKV_ERR_INVALID_ARG, "at most 65535 pairs per call");
  const int64_t E = pkv::elem_bytes(cfg->dtype);
  const int64_t slab = int64_t(cfg->num_kv_heads) * pkv::tile_elems(*cfg) * E;
  const int64_t layer_bytes = pkv::layer_elems(*cfg) * E;
  dim3 grid(n, cfg->num_layers, 3);
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<char*>(pool_dev), pairs_dev, cfg->num_blocks, slab, layer_bytes,
                     pkv::region_bytes(*cfg), int64_t(cfg->num_kv_heads) * 2 * 2, cfg->dtype == PKV_I8 ? 1 : 0);
  return hip_status(hipGetLastError(), "copy_blocks launch");
}

int pkv_append_kv(const pkv_config* cfg, void* pool_dev, int32_t layer, const void* k_dev, const void* v_dev,
                  const int32_t* slots_dev, int32_t n_tokens, void* stream) {
  int st = pkv::validate_config(cfg);
  if (st != PKV_OK) return st;
  if (layer < 0 || layer >= cfg->num_layers) return pkv::fail(PKV_ERR_INVALID_ARG, "layer %d out of range", layer);
  if (n_tokens < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "n_tokens must be >= 0");
  if (n_tokens == 0) return PKV_OK;
  if (!pool_dev || !k_dev || !v_dev || !slots_dev) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL device pointer");
  if (!aligned16(pool_dev) || !aligned16(k_dev) || !aligned16(v_dev))
    return pkv::fail(PKV_ERR_INVALID_ARG, "pool, k and v must be 16-byte aligned");
  if (cfg->dtype == PKV_I8) {
    if (n_tokens > INT32_MAX / 2) return pkv::fail(PKV_ERR_INVALID_ARG, "too many tokens in one call");
    if (cfg->num_kv_heads > 65535) return pkv::fail(PKV_ERR_UNSUPPORTED, "too many KV heads");
    const int64_t layer_bytes = pkv::layer_elems(*cfg);
    char* base = static_cast<char*>(pool_dev);
    int8_t* Kl = reinterpret_cast<int8_t*>(base + layer * layer_bytes);
    int8_t* Vl = reinterpret_cast<int8_t*>(base + pkv::region_bytes(*cfg) + layer * layer_bytes);
    _Float16* Sl = reinterpret_cast<_Float16*>(base + 2 * pkv::region_bytes(*cfg) +
                                               int64_t(layer) * cfg->num_blocks * cfg->num_kv_heads * 2 * 2);
    const dim3 grid(unsigned(n_tokens), unsigned(cfg->num_kv_heads), 2);
    auto kern = cfg->head_dim == 128 ? append_kv_i8_kernel<128> : append_kv_i8_kernel<64>;
    hipLaunchKernelGGL(kern, grid, dim3(64), 0, static_cast<hipStream_t>(stream), Kl, Vl, Sl,
                       static_cast<const _Float16*>(k_dev), static_cast<const _Float16*>(v_dev), slots_dev,
                       n_tokens, cfg->num_kv_heads, cfg->num_blocks);
    return hip_status(hipGetLastError(), "append_kv launch");
  }
  const int64_t layer_bytes = pkv::layer_elems(*cfg) * 2;
  char* base = static_cast<char*>(pool_dev);
  uint4* Kl = reinterpret_cast<uint4*>(base + layer * layer_bytes);
  uint4* Vl = reinterpret_cast<uint4*>(base + pkv::region_bytes(*cfg) + layer * layer_bytes);
  const int64_t threads = int64_t(n_tokens) * cfg->num_kv_heads * (cfg->head_dim / 8);
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > INT32_MAX) return pkv::fail(PKV_ERR_INVALID_ARG, "too many tokens in one call");
  hipLaunchKernelGGL(append_kv_f16_kernel, dim3(unsigned(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     Kl, Vl, static_cast<const uint4*>(k_dev), static_cast<const uint4*>(v_dev), slots_dev,
                     n_tokens, cfg->num_kv_heads, cfg->head_dim, cfg->num_blocks);
  return hip_status(hipGetLastError(), "append_kv launch");
}

int64_t pkv_decode_workspace_bytes(const pkv_config* cfg, int32_t num_seqs, int32_t num_q_heads,
                                   int32_t max_context, int32_t partition_tokens) {
  int st = pkv::validate_config(cfg);
  if (st != PKV_OK) return st;
  if (num_seqs < 1 || num_q_heads < 1 || max_context < 1)
    return pkv::fail(PKV_ERR_INVALID_ARG, "num_seqs, num_q_heads and max_context must be >= 1");
  st = check_partition_tokens(partition_tokens);
  if (st != PKV_OK) return st;
  return ws_layout(*cfg, num_seqs, num_q_heads, max_context, 1, partition_tokens, 0).bytes;
}

}  // extern "C"

namespace {

// Scratch of pkv_paged_decode_noalloc: the split-K partials of a decode, in
// a file-scope device array (one copy per GPU the library runs on, held
// until the process ends). Its address on a device comes from
// hipGetSymbolAddress, taken once per device with that device current; host
// code never passes the array's name itself to a kernel or a copy.
constexpr int64_t NOALLOC_SCRATCH_BYTES = PKV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[NOALLOC_SCRATCH_BYTES];

int scratch_on_current_device(void** out) {
  static std::mutex mu;
  static std::map<int, void*> known;
  int dev = 0;
  int st = hip_status(hipGetDevice(&dev), "hipGetDevice");
  if (st != PKV_OK) return st;
  std::lock_guard<std::mutex> lock(mu);
  const auto it = known.find(dev);
  if (it != known.end()) {
    *out = it->second;
    return PKV_OK;
  }
  void* ptr = nullptr;
  st = hip_status(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
  if (st != PKV_OK) return st;
  known[dev] = ptr;
  *out = ptr;
  return PKV_OK;
}

int paged_decode_impl(const pkv_decode_args* a, void* stream, void* ws_dev, int64_t ws_bytes, bool noalloc) {
  if (!a) return pkv::fail(PKV_ERR_INVALID_ARG, "args is NULL");
  int st = pkv::validate_config(a->cfg);
  if (st != PKV_OK) return st;
  const pkv_config& c = *a->cfg;
  if (!a->pool_dev || !a->q_dev || !a->block_tables_dev || !a->ctx_lens_dev || !a->out_dev)
    return pkv::fail(PKV_ERR_INVALID_ARG, "NULL device pointer");
  if (!aligned16(a->pool_dev) || !aligned16(a->q_dev))
    return pkv::fail(PKV_ERR_INVALID_ARG, "pool and q must be 16-byte aligned");
  if (a->layer < 0 || a->layer >= c.num_layers)
    return pkv::fail(PKV_ERR_INVALID_ARG, "layer %d out of range", a->layer);
  if (a->num_seqs < 1 || a->num_seqs > 65535) return pkv::fail(PKV_ERR_INVALID_ARG, "num_seqs must be in [1, 65535]");
  if (a->num_q_heads < 1 || a->num_q_heads % c.num_kv_heads)
    return pkv::fail(PKV_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d", a->num_q_heads,
                     c.num_kv_heads);
  if (a->max_blocks < 1 || a->max_context < 1)
    return pkv::fail(PKV_ERR_INVALID_ARG, "max_blocks and max_context must be >= 1");
  st = check_partition_tokens(a->partition_tokens);
  if (st != PKV_OK) return st;
  if ((a->k_new_dev == nullptr) != (a->v_new_dev == nullptr))
    return pkv::fail(PKV_ERR_INVALID_ARG, "k_new and v_new must both be given or both be NULL");
  if (a->k_new_dev && (!aligned16(a->k_new_dev) || !aligned16(a->v_new_dev)))
    return pkv::fail(PKV_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
  const int G = a->num_q_heads / c.num_kv_heads;
  const int kg = G <= 2 ? G : G <= 4 ? 4 : 8;  // the group size the kernel is built for
  decode_fn fn = pick_kernel(c.head_dim, G, c.dtype == PKV_I8, a->prefix_groups > 0 ? GRID_PLAN : GRID_PLAIN);
  if (!fn) return pkv::fail(PKV_ERR_UNSUPPORTED, "group size %d not built (1 to 8)", G);
  if (c.num_kv_heads > 65535) return pkv::fail(PKV_ERR_UNSUPPORTED, "too many KV heads");
  if (a->ctx_lens_host) {
    const int64_t cap = std::min<int64_t>(int64_t(a->max_blocks) * BT, a->max_context);
    for (int b = 0; b < a->num_seqs; ++b) {
      const int32_t n = a->ctx_lens_host[b];
      if (n < 1 || n > cap)
        return pkv::fail(PKV_ERR_INVALID_ARG, "context_len[%d] = %d outside [1, %lld]", b, n, (long long)cap);
    }
  }
  // shared-prefix plan
  const bool plan = a->prefix_groups > 0;
  if (a->prefix_groups < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "prefix_groups must be >= 0");
  if (plan && !a->prefix_plan_dev) return pkv::fail(PKV_ERR_INVALID_ARG, "prefix_groups > 0 needs prefix_plan_dev");
  if (plan && a->prefix_groups > a->num_seqs / 2)
    return pkv::fail(PKV_ERR_INVALID_ARG, "more groups (%d) than pairs of sequences", a->prefix_groups);
  if (plan && a->prefix_plan_host) {
    const int32_t* ph = a->prefix_plan_host;
    const int B = a->num_seqs;
    for (int gi = 0; gi < a->prefix_groups; ++gi) {
      const int32_t* gd = ph + 2 * int64_t(B) + int64_t(gi) * PKV_PREFIX_GROUP_INTS;
      if (gd[0] < 1 || gd[0] > a->max_blocks || gd[1] < 2 || gd[1] > PKV_MAX_SHARERS || gd[1] * G > PREFIX_ROWS)
        return pkv::fail(PKV_ERR_INVALID_ARG, "plan group %d: %d blocks, %d members (members x %d heads <= %d)", gi,
                         gd[0], gd[1], G, PREFIX_ROWS);
      for (int m = 0; m < gd[1]; ++m) {
        const int bb = gd[2 + m];
        if (bb < 0 || bb >= B || ph[2 * bb + 1] != gi * 64 + m || ph[2 * bb] != gd[0])
          return pkv::fail(PKV_ERR_INVALID_ARG, "plan group %d member %d is inconsistent", gi, m);
        if (a->ctx_lens_host && (a->ctx_lens_host[bb] - 1) / BT < gd[0])
          return pkv::fail(PKV_ERR_INVALID_ARG, "plan group %d shares the block of a member's last token", gi);
      }
    }
  }

  const WsLayout wl =
      ws_layout(c, a->num_seqs, a->num_q_heads, a->max_context, a->max_blocks, a->partition_tokens, a->prefix_groups);
  const int mp0 = wl.grid_parts, mp = wl.max_parts;
  const int64_t need = wl.bytes;
  if (noalloc && need > ws_bytes)
    return pkv::fail(PKV_ERR_INVALID_ARG,
                     "pkv_paged_decode_noalloc: this decode needs %lld bytes of split-K scratch, above its "
                     "maximum of %lld (use pkv_paged_decode with a workspace)",
                     (long long)need, (long long)ws_bytes);
  if (need > 0 && (!ws_dev || ws_bytes < need))
    return pkv::fail(PKV_ERR_INVALID_ARG, "workspace too small: need %lld bytes", (long long)need);
  if (need > 0 && !aligned16(ws_dev))
    return pkv::fail(PKV_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  // prefix partitions of this launch: the workspace's count, or fewer when
  // the plan's host copy shows shorter shared runs
  int pp = wl.prefix_pp, pz = wl.prefix_z;
  if (plan && a->prefix_plan_host) {
    int max_np = 1;
    for (int gi = 0; gi < a->prefix_groups; ++gi)
      max_np = std::max(max_np, std::min(a->prefix_plan_host[2 * int64_t(a->num_seqs) +
                                                           int64_t(gi) * PKV_PREFIX_GROUP_INTS],
                                         a->max_blocks));
    pp = std::min(pp, std::max(1, (max_np + PREFIX_PART_BLOCKS - 1) / PREFIX_PART_BLOCKS));
    pz = int((int64_t(pp) * a->prefix_groups * PREFIX_SPLIT + a->num_seqs - 1) / a->num_seqs);
  }
  if (int64_t(pz) + mp0 > 65535) return pkv::fail(PKV_ERR_UNSUPPORTED, "too many partitions for one launch");

  // Partition size of this launch, unless the caller fixed it.
  // - Without a plan: the one-round rule over each sequence's blocks (every
  //   sequence at max_context when the host lengths are not given), never
  //   finer than the workspace's cut, so that the grid covers max_context
  //   within the workspace's partial rows.
  // - With a plan and both host copies: the longest stretch the split role
  //   covers (a grouped sequence's unshared tail, an ungrouped sequence's
  //   whole context) cut for about 2048 work-groups (512 for int8), in at
  //   most as many partitions as the grid and the workspace hold. The
  //   shared-prefix work-groups are the launch's longest chains, and split
  //   work-groups cut this finely finish beside them (32 sequences over a
  //   2048-token prefix: 22.7 us, against 23.7 us with the one-round rule).
  int pb = wl.part_blocks, gparts = mp0;
  if (a->partition_tokens == 0 && !std::getenv("PKV_PARTITION_TOKENS")) {
    if (!plan) {
      const int64_t cap = std::min<int64_t>(int64_t(a->max_blocks) * BT, a->max_context);
      const int cap_blocks = int((cap + BT - 1) / BT);
      const int32_t* lens = a->ctx_lens_host;
      auto span = [&](int b) { return lens ? int((std::min<int64_t>(lens[b], cap) + BT - 1) / BT) : cap_blocks; };
      pb = launch_part_blocks(c.num_kv_heads, a->num_seqs, span,
                              resident_wgs(reinterpret_cast<const void*>(fn),
                                           decode_dyn_lds(reinterpret_cast<const void*>(fn), c.dtype == PKV_I8, kg,
                                                          plan ? GRID_PLAN : GRID_PLAIN)),
                              (cap_blocks + mp0 - 1) / mp0);
      gparts = std::min(mp0, (cap_blocks + pb - 1) / pb);
    } else if (a->ctx_lens_host && a->prefix_plan_host) {
      int span = 1;
      for (int b = 0; b < a->num_seqs; ++b) {
        const int nb = (a->ctx_lens_host[b] + BT - 1) / BT;
        span = std::max(span, nb - std::max(0, std::min(a->prefix_plan_host[2 * b], a->max_blocks)));
      }
      pb = std::max(choose_part_blocks(c.num_kv_heads, a->num_seqs, span * BT, 0, c.dtype == PKV_I8 ? 512 : 2048),
                    (span + mp0 - 1) / mp0);
    }
  }

  // Stream-K split (host lengths given, automatic partitions): the spans the
  // split role covers (every block without a plan; a grouped sequence's
  // blocks after its shared ones with one) laid end to end and cut into
  // equal runs of q blocks per work-group, about one round of resident
  // work-groups beside the shared-prefix ones. Without a plan it is taken
  // for ragged batches, whose plain grid would launch work-groups past some
  // sequence's last partition: the plain grid's cut leaves short remainder
  // partitions beside full ones, and the longest work-groups set the launch
  // time; equal runs leave none longer than q (the continuous-batching mix:
  // 72 blocks at most, against 81 for the one-round partitions; 53.0 ->
  // 51.4 us). With a plan (and its host copy) it always is: the plain
  // grid's split planes queue behind work-groups with nothing to do.
  const int units = plan ? pp * a->prefix_groups * PREFIX_SPLIT : 0;  // prefix work-groups per KV head
  bool stream_k = false;
  int64_t stream_wgs = 0;
  int stream_rows = 0;
  if (a->ctx_lens_host && (!plan || a->prefix_plan_host) && a->num_seqs <= STREAM_MAX_SEQS &&
      a->partition_tokens == 0 && !std::getenv("PKV_PARTITION_TOKENS")) {
    const int64_t cap = std::min<int64_t>(int64_t(a->max_blocks) * BT, a->max_context);
    auto shared = [&](int b) {
      return plan ? std::min(std::max(a->prefix_plan_host[2 * b], 0), a->max_blocks) : 0;
    };
    auto pre_parts = [&](int b) {  // the prefix partials leading sequence b's row
      if (!plan) return 0;
      const int sb = shared(b), gm = a->prefix_plan_host[2 * b + 1];
      if (gm < 0 || (gm >> 6) >= a->prefix_groups || sb <= 0) return 0;
      const int pbp = (sb + pp - 1) / pp;
      return (sb + pbp - 1) / pbp;
    };
    const int pad = stream_pad_blocks(c.dtype);
    int64_t pairs = 0, T = 0;
    for (int b = 0; b < a->num_seqs; ++b) {
      const int64_t nb = std::max<int64_t>((std::min<int64_t>(a->ctx_lens_host[b], cap) + BT - 1) / BT - shared(b), 0);
      pairs += (nb + pb - 1) / pb;
      T += nb > 0 ? nb + pad : 0;
    }
    if ((plan || pairs < int64_t(a->num_seqs) * gparts) && T > 0) {
      // the residency of the kernel that will run the cut (the stream-K one without a plan)
      const void* sk = plan ? reinterpret_cast<const void*>(fn)
                            : reinterpret_cast<const void*>(pick_kernel(c.head_dim, G, c.dtype == PKV_I8, GRID_STREAM));
      const Residency res = resident_wgs(sk, decode_dyn_lds(sk, c.dtype == PKV_I8, kg, plan ? GRID_PLAN : GRID_STREAM));
      const int64_t slots_h = std::max<int64_t>(1, res.slots / c.num_kv_heads - units);
      int64_t q = (T + slots_h - 1) / slots_h;
      q = std::min<int64_t>(std::max<int64_t>(q, MIN_PART_BLOCKS), MAX_PARTITION_TOKENS / BT);
      int64_t cb = 0;  // where sequence b's charge starts in the run
      int rows_max = 0;
      for (int b = 0; b < a->num_seqs; ++b) {
        const int64_t nb =
            std::max<int64_t>((std::min<int64_t>(a->ctx_lens_host[b], cap) + BT - 1) / BT - shared(b), 0);
        if (nb == 0) continue;
        const int64_t first = cb + pad;  // its first real block
        rows_max = std::max<int>(rows_max, pre_parts(b) + int((first + nb - 1) / q - first / q + 1));
        cb = first + nb;
      }
      if (rows_max <= mp && (T + q - 1) / q + units <= int64_t(65535) * 65535) {
        stream_k = true;
        stream_wgs = (T + q - 1) / q;
        stream_rows = rows_max;
        pb = int(q);
      }
    }
  }

  const int64_t E = pkv::elem_bytes(c.dtype);
  const int64_t layer_bytes = pkv::layer_elems(c) * E;
  const char* base = static_cast<const char*>(a->pool_dev);
  DecodeParams prm;
  prm.K = base + a->layer * layer_bytes;
  prm.V = base + pkv::region_bytes(c) + a->layer * layer_bytes;
  prm.scales = c.dtype == PKV_I8
                   ? reinterpret_cast<const _Float16*>(base + 2 * pkv::region_bytes(c) +
                                                     int64_t(a->layer) * c.num_blocks * c.num_kv_heads * 2 * 2)
                   : nullptr;
  prm.q = static_cast<const _Float16*>(a->q_dev);
  prm.k_new = static_cast<const uint4*>(a->k_new_dev);
  prm.v_new = static_cast<const uint4*>(a->v_new_dev);
  prm.tables = a->block_tables_dev;
  prm.ctx_lens = a->ctx_lens_dev;
  const int64_t rows = int64_t(a->num_seqs) * a->num_q_heads * mp;
  float* ws = static_cast<float*>(ws_dev);
  const bool parts = need > 0;
  prm.part_m = parts ? ws : nullptr;
  prm.part_l = parts ? ws + rows : nullptr;
  prm.part_o = parts ? ws + 2 * rows : nullptr;
  prm.out = static_cast<_Float16*>(a->out_dev);
  prm.plan = plan ? a->prefix_plan_dev : nullptr;
  prm.prefix_z = pz;
  prm.prefix_pp = pp;
  prm.num_groups = plan ? a->prefix_groups : 0;
  prm.max_blocks = a->max_blocks;
  prm.num_blocks = c.num_blocks;
  prm.Hkv = c.num_kv_heads;
  prm.part_blocks = pb;
  prm.max_parts = mp;
  prm.max_context = a->max_context;
  prm.scale_log2 = a->scale * LOG2E;
  prm.num_seqs = a->num_seqs;
  prm.plan_stream = plan && stream_k ? 1 : 0;
  prm.stream_pad = stream_k ? stream_pad_blocks(c.dtype) : 0;
  prm.group = G;
  if (stream_k && !plan) fn = pick_kernel(c.head_dim, G, c.dtype == PKV_I8, GRID_STREAM);

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
  if (a->timing_events)
    for (int i = 0; i < 4; ++i) ev[i] = static_cast<hipEvent_t>(a->timing_events[i]);

  // The fused append (if any) writes into private tail blocks only, which no
  // shared-prefix work-group reads.
  const int64_t lin = stream_wgs + units;  // stream-K: prefix work-groups first, then the runs
  const int cy = int(std::min<int64_t>(lin, 65535));
  const dim3 grid = stream_k ? dim3(c.num_kv_heads, cy, unsigned((lin + cy - 1) / cy))
                             : dim3(c.num_kv_heads, a->num_seqs, pz + gparts);
  const size_t dyn_lds = decode_dyn_lds(reinterpret_cast<const void*>(fn), c.dtype == PKV_I8, kg,
                                        plan ? GRID_PLAN : (stream_k ? GRID_STREAM : GRID_PLAIN));
  if (ev[0] && ev[1])
    hipExtLaunchKernelGGL(fn, grid, dim3(256), dyn_lds, s, ev[0], ev[1], 0, prm);
  else
    hipLaunchKernelGGL(fn, grid, dim3(256), dyn_lds, s, prm);
  st = hip_status(hipGetLastError(), "paged_decode launch");
  if (st != PKV_OK || (stream_k ? stream_rows <= 1 && !plan : gparts <= 1 && !plan)) return st;
  MergeParams mg;
  mg.part_m = prm.part_m;
  mg.part_l = prm.part_l;
  mg.part_o = prm.part_o;
  mg.ctx_lens = a->ctx_lens_dev;
  mg.plan = prm.plan;
  mg.out = prm.out;
  mg.D = c.head_dim;
  mg.max_blocks = a->max_blocks;
  mg.max_context = a->max_context;
  mg.part_blocks = pb;
  mg.max_parts = mp;
  mg.num_groups = prm.num_groups;
  mg.prefix_pp = prm.prefix_pp;
  mg.row_parts = stream_k ? stream_rows : std::min(mp, (plan ? pp : 0) + gparts);
  mg.num_seqs = a->num_seqs;
  mg.stream_q = stream_k ? pb : 0;
  mg.stream_pad = prm.stream_pad;
  const dim3 rgrid(a->num_q_heads, a->num_seqs);
  const int ways = merge_ways(mg.row_parts);
  if (ev[2] && ev[3])
    hipExtLaunchKernelGGL(lse_reduce_kernel, rgrid, dim3(c.head_dim, ways), 0, s, ev[2], ev[3], 0, mg);
  else
    hipLaunchKernelGGL(lse_reduce_kernel, rgrid, dim3(c.head_dim, ways), 0, s, mg);
  return hip_status(hipGetLastError(), "lse_reduce launch");
}

}  // namespace

extern "C" {

int pkv_paged_decode(const pkv_decode_args* a, void* stream) {
  if (!a) return pkv::fail(PKV_ERR_INVALID_ARG, "args is NULL");
  return paged_decode_impl(a, stream, a->workspace_dev, a->workspace_bytes, false);
}

int pkv_paged_decode_noalloc(const pkv_decode_args* a, void* stream) {
  if (!a) return pkv::fail(PKV_ERR_INVALID_ARG, "args is NULL");
  void* ptr = nullptr;
  const int st = scratch_on_current_device(&ptr);
  if (st != PKV_OK) return st;
  return paged_decode_impl(a, stream, ptr, NOALLOC_SCRATCH_BYTES, true);
}

int pkv_paged_prefill(const pkv_prefill_args* a, void* stream) {
  if (!a) return pkv::fail(PKV_ERR_INVALID_ARG, "args is NULL");
  int st = pkv::validate_config(a->cfg);
  if (st != PKV_OK) return st;
  const pkv_config& c = *a->cfg;
  if (a->num_seqs < 1 || a->num_seqs > 65535) return pkv::fail(PKV_ERR_INVALID_ARG, "num_seqs must be in [1, 65535]");
  if (!a->q_start_host) return pkv::fail(PKV_ERR_INVALID_ARG, "q_start_host is required");
  const int32_t* qs = a->q_start_host;
  if (qs[0] != 0) return pkv::fail(PKV_ERR_INVALID_ARG, "q_start[0] must be 0");
  int max_ql = 0;
  for (int b = 0; b < a->num_seqs; ++b) {
    const int ql = qs[b + 1] - qs[b];
    if (ql < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "q_start must not decrease (sequence %d)", b);
    max_ql = std::max(max_ql, ql);
  }
  if (max_ql == 0) return PKV_OK;  // no query rows
  if (!a->pool_dev || !a->q_dev || !a->q_start_dev || !a->block_tables_dev || !a->ctx_lens_dev || !a->out_dev)
    return pkv::fail(PKV_ERR_INVALID_ARG, "NULL device pointer");
  if (!aligned16(a->pool_dev) || !aligned16(a->q_dev) || !aligned16(a->out_dev))
    return pkv::fail(PKV_ERR_INVALID_ARG, "pool, q and out must be 16-byte aligned");
  if (a->layer < 0 || a->layer >= c.num_layers) return pkv::fail(PKV_ERR_INVALID_ARG, "layer %d out of range", a->layer);
  if (a->num_q_heads < 1 || a->num_q_heads % c.num_kv_heads)
    return pkv::fail(PKV_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d", a->num_q_heads,
                     c.num_kv_heads);
  if (a->max_blocks < 1 || a->max_context < 1)
    return pkv::fail(PKV_ERR_INVALID_ARG, "max_blocks and max_context must be >= 1");
  const int G = a->num_q_heads / c.num_kv_heads;
  if (c.num_kv_heads > 65535) return pkv::fail(PKV_ERR_UNSUPPORTED, "too many KV heads");
  if (a->ctx_lens_host) {
    const int64_t cap = std::min<int64_t>(int64_t(a->max_blocks) * BT, a->max_context);
    for (int b = 0; b < a->num_seqs; ++b) {
      const int32_t n = a->ctx_lens_host[b];
      if (n < 1 || n > cap)
        return pkv::fail(PKV_ERR_INVALID_ARG, "context_len[%d] = %d outside [1, %lld]", b, n, (long long)cap);
      if (qs[b + 1] - qs[b] > n)
        return pkv::fail(PKV_ERR_INVALID_ARG, "sequence %d: %d query tokens but %d cached", b, qs[b + 1] - qs[b], n);
    }
  }
  typedef void (*fn_t)(PrefillParams);
  fn_t fn = nullptr;
  const bool i8 = c.dtype == PKV_I8;
  // group sizes 1, 2, 4 and 8 have kernels of their own; 3, 5, 6 and 7 take
  // theirs at run time (G = 0)
  const bool own = G == 1 || G == 2 || G == 4 || G == 8, any = G >= 1 && G <= 8;
  if (c.head_dim == 128) {
    fn = G == 1 ? (i8 ? prefill_kernel<128, 1, true> : prefill_kernel<128, 1, false>)
       : G == 2 ? (i8 ? prefill_kernel<128, 2, true> : prefill_kernel<128, 2, false>)
       : G == 4 ? (i8 ? prefill_kernel<128, 4, true> : prefill_kernel<128, 4, false>)
       : G == 8 ? (i8 ? prefill_kernel<128, 8, true> : prefill_kernel<128, 8, false>)
       : any && !own ? (i8 ? prefill_kernel<128, 0, true> : prefill_kernel<128, 0, false>) : nullptr;
  } else if (c.head_dim == 64) {
    fn = G == 1 ? (i8 ? prefill_kernel<64, 1, true> : prefill_kernel<64, 1, false>)
       : G == 2 ? (i8 ? prefill_kernel<64, 2, true> : prefill_kernel<64, 2, false>)
       : G == 4 ? (i8 ? prefill_kernel<64, 4, true> : prefill_kernel<64, 4, false>)
       : G == 8 ? (i8 ? prefill_kernel<64, 8, true> : prefill_kernel<64, 8, false>)
       : any && !own ? (i8 ? prefill_kernel<64, 0, true> : prefill_kernel<64, 0, false>) : nullptr;
  }
  if (!fn) return pkv::fail(PKV_ERR_UNSUPPORTED, "group size %d not built (1 to 8)", G);
  const int QT = PREFIX_ROWS / G;
  const int qtiles = (max_ql + QT - 1) / QT;
  const int pairs = (qtiles + 1) / 2;  // each work-group takes a long and a short query tile
  if (pairs > 65535) return pkv::fail(PKV_ERR_UNSUPPORTED, "chunk too long");

  const int64_t layer_bytes = pkv::layer_elems(c) * pkv::elem_bytes(c.dtype);
  const char* base = static_cast<const char*>(a->pool_dev);
  PrefillParams prm;
  prm.K = base + a->layer * layer_bytes;
  prm.V = base + pkv::region_bytes(c) + a->layer * layer_bytes;
  prm.q = static_cast<const _Float16*>(a->q_dev);
  prm.q_start = a->q_start_dev;
  prm.tables = a->block_tables_dev;
  prm.ctx_lens = a->ctx_lens_dev;
  prm.out = static_cast<_Float16*>(a->out_dev);
  prm.scales = i8 ? reinterpret_cast<const uint32_t*>(base + 2 * pkv::region_bytes(c) +
                                                     int64_t(a->layer) * c.num_blocks * c.num_kv_heads * 2 * 2)
                  : nullptr;
  prm.Hkv = c.num_kv_heads;
  prm.max_blocks = a->max_blocks;
  prm.num_blocks = c.num_blocks;
  prm.max_context = a->max_context;
  prm.scale_log2 = a->scale * LOG2E;
  prm.group = G;
  hipLaunchKernelGGL(fn, dim3(c.num_kv_heads, pairs, a->num_seqs), dim3(256), 0, static_cast<hipStream_t>(stream),
                     prm);
  return hip_status(hipGetLastError(), "paged_prefill launch");
}

int64_t pkv_prefix_decode_workspace_bytes(const pkv_config* cfg, int32_t num_seqs, int32_t num_q_heads,
                                          int32_t max_context, int32_t max_blocks, int32_t partition_tokens,
                                          int32_t n_groups) {
  int st = pkv::validate_config(cfg);
  if (st != PKV_OK) return st;
  if (num_seqs < 1 || num_q_heads < 1 || max_context < 1 || max_blocks < 1 || n_groups < 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "num_seqs, num_q_heads, max_context, max_blocks >= 1, n_groups >= 0");
  st = check_partition_tokens(partition_tokens);
  if (st != PKV_OK) return st;
  return ws_layout(*cfg, num_seqs, num_q_heads, max_context, max_blocks, partition_tokens, n_groups).bytes;
}

int pkv_upload(void* dst_dev, const void* src_host, int64_t bytes, void* stream) {
  if (bytes < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "bytes must be >= 0");
  if (bytes == 0) return PKV_OK;
  if (!dst_dev || !src_host) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(dst_dev) || !aligned16(src_host))
    return pkv::fail(PKV_ERR_INVALID_ARG, "dst and src must be 16-byte aligned");
  // The kernel reads src through the device mapping of pinned host memory:
  // anything else (pageable memory, device memory) is refused here, before
  // any launch.
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, src_host) != hipSuccess || attr.type != hipMemoryTypeHost ||
      attr.devicePointer == nullptr) {
    (void)hipGetLastError();  // clear the sticky error of a failed query
    return pkv::fail(PKV_ERR_INVALID_ARG, "src_host is not pinned host memory mapped for the device");
  }
  hipPointerAttribute_t dattr;
  if (hipPointerGetAttributes(&dattr, dst_dev) != hipSuccess || dattr.type != hipMemoryTypeDevice) {
    (void)hipGetLastError();
    return pkv::fail(PKV_ERR_INVALID_ARG, "dst_dev is not device memory");
  }
  const int64_t n16 = bytes / 16;
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((n16 + 255) / 256, 1024));
  hipLaunchKernelGGL(upload_kernel, dim3(unsigned(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<char*>(dst_dev), static_cast<const char*>(attr.devicePointer), bytes);
  return hip_status(hipGetLastError(), "upload launch");
}


int pkv_probe_stream_read(const void* buf_dev, int64_t bytes, void* sink_dev, void* stream) {
  if (!buf_dev || !sink_dev || bytes < 16 || !aligned16(buf_dev))
    return pkv::fail(PKV_ERR_INVALID_ARG, "bad probe arguments");
  hipLaunchKernelGGL(stream_read_kernel, dim3(256 * 16), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(buf_dev), bytes / 16, static_cast<uint32_t*>(sink_dev));
  return hip_status(hipGetLastError(), "stream_read launch");
}

}  // extern "C"
