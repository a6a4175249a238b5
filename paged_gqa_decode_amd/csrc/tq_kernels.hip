// gfx950 (CDNA4) kernels of paged grouped-query decode attention over a
// quantized KV cache (fp8 e4m3fn codes with per-row fp32 scales, or the 4-bit
// record of centroid-coded K and affine V), and the writer that fills the fp8
// cache.  The file holds, in order: the fp8 token stream and the 4-bit token
// stream (the per-wave cores every decode kernel runs), the split-K partition
// kernel, the per-(s, h) fused kernel, the flat even-split fused kernel, the
// log-sum-exp merge of the partition kernel's partials, the KV-cache writer,
// and the host launchers.
//
// What is computed follows the page "vllm.v1.attention.ops.flydsl_kernels.
// tq_decode": the block-table walk (STEP F), the QK^T and PV products with
// the query group on the MFMA's 16 columns, the online softmax with running
// max and sum (STEP F, FA-2 state of STEP D), and the normalised partial
// output with its max logit and exp sum (STEP G).  The kernel design here is
// its own, made for gfx950 (for the fp8 stream; the 4-bit stream is
// described where it is defined):
//
//  * One 64-lane wave walks a run of tokens of one (sequence s, kv head h) as
//    one stream of 32-token chunks (two 16-token MFMA tiles), with the next
//    chunk's loads in flight while the current one is computed.  At every
//    boundary its caller asks for (a split-K partition, a tile group), the
//    finished partial goes to the caller and the softmax state restarts, so a
//    partial does not depend on how runs are dealt to waves.
//  * K never touches LDS.  QK^T contracts over head_dim, so any permutation
//    of d applied to both q and K is allowed: lane (r = lane%16, b = lane/16)
//    supplies K[token r][d = 32b .. 32b+31], one contiguous 32-byte piece of
//    the token's 128-byte row (two 16-byte loads), and q is loaded with the
//    same permutation.  fp8 e4m3fn -> bf16 is exact, so the MFMA sees the
//    exact codes; the per-token K scale and softmax_scale*log2(e) multiply
//    the fp32 logits afterwards.
//  * V and the K/V scales go HBM -> LDS directly (global_load_lds_dwordx4 /
//    _dword, no VGPRs), V rows stored with their 16-byte pieces XOR-swizzled.
//    ds_read_b64_tr_b8 then returns, per lane, 8 tokens of one head_dim
//    column: the A operand of a 16x16x32 f16 MFMA (O^T = V^T P), converted
//    fp8 -> f16 exactly in registers.
//  * The V scale is folded into P: the B operand is p_t * vs_t / sigma in
//    f16, where sigma is the running maximum |V scale| since the last restart,
//    so the operand stays in [-1, 1] whatever the data's magnitude or sign;
//    acc is rescaled when sigma grows, together with the softmax rescale.
//  * Tokens past the sequence end inside the last chunk may hold any bytes
//    (NaN codes or scales included): their logits are selected to -inf, their
//    P and V operand bytes to zero, so they cannot reach the result.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "tq_internal.h"

namespace tq {

// The static scratch of tq_decode_fused_static (device memory each GPU holds
// until the process ends): arrival counters in the first kStaticCounterBytes,
// workgroup partials after them.  Host code never passes this name to a
// kernel; it takes the device address from static_scratch().
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int D = kHeadDim;
constexpr int CHUNK = 32;  // tokens per pipeline step
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309417f;

// Cache policy of the LDS-direct loads: the NT (non-temporal, streaming) bit
// of gfx940-family cache-policy operands.  Every KV byte is read once; with
// NT the V / scale stream measured 8-9% faster on the bandwidth workload.
constexpr int kCachePolicyStreaming = 2;
// Word 3 of a gfx9 buffer resource for raw (untyped) buffer loads and stores.
constexpr int kBufferDword3 = 0x00020000;

// s_waitcnt with vmcnt = 0 and the other counters left at their maxima
// (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]).
constexpr int kWaitVmcnt0 = (0x7 << 4) | (0xF << 8);

// max(a, b) for operands that are not NaN, as one v_med3_f32 against +inf:
// fmaxf would first quiet each operand that the compiler cannot prove is no
// signalling NaN (every value that comes from another lane or from memory),
// one extra instruction per operand.
__device__ __forceinline__ float fmax_nn(float a, float b) {
  // +inf from an opaque scalar move, or the compiler folds the median back
  // into a maximum and reinstates the quieting.
  float inf;
  asm("s_mov_b32 %0, 0x7f800000" : "=s"(inf));
  return __builtin_amdgcn_fmed3f(a, b, inf);
}

// Reductions over the lanes l, l^16, l^32, l^48 (the four 16-lane groups) by
// the gfx950 lane swaps, no LDS round trip: v_permlane16_swap of a value with
// itself leaves {own, partner l^16} in the two results (in some order), and
// v_permlane32_swap {own, partner l^32}.  Max and sum are commutative, so
// every lane gets the same bits, as with a pair of xor shuffles.
__device__ __forceinline__ float wave_max_xor16_32(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmax_nn(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmax_nn(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

// Maximum over all 64 lanes: rotations by 8, 4, 2, 1 within each 16-lane row
// (DPP row_ror), then across the rows.
__device__ __forceinline__ float wave_max_all(float x) {
  x = fmax_nn(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false)));
  x = fmax_nn(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false)));
  x = fmax_nn(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false)));
  x = fmax_nn(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false)));
  return wave_max_xor16_32(x);
}

__device__ __forceinline__ float wave_sum_xor16_32(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Sum over all 64 lanes: rotations by 8, 4, 2, 1 within each 16-lane row,
// then across the rows.  The lanes add in different orders, so lane 0's sum is
// broadcast: every lane returns the same bits.
__device__ __forceinline__ float wave_sum_all(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false));
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wave_sum_xor16_32(x))));
}

// x of lane r + 8 (mod 16) of the same 16-lane row (DPP row_ror:8).
__device__ __forceinline__ float row_ror8(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), 0x128, 0xF, 0xF, false));
}

// The 4-bit stream's softmax runs on 4 tokens per lane instead of 8 when the
// query group fits in 8 MFMA columns (lanes r >= 8 then hold the second tile).
constexpr bool tq4_compact_softmax(int QG) { return QG <= 8; }

// 8 fp8 e4m3fn codes (two dwords) -> 8 bf16, exact.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(int w0, int w1) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// 8 fp8 e4m3fn codes (two dwords) -> 8 f16, exact.
__device__ __forceinline__ f16x8 fp8x8_to_f16(int w0, int w1) {
  f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
  f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
  f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
  f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Byte offset, inside its block, of the 128-byte row of (kv head h, slot): the
// rows are head-major or slot-major (the page's data-region order) as the two
// strides say.  Below 2^31 (a block holds Hkv*BS rows of 128 bytes).
__device__ __forceinline__ uint32_t row_in_block(const StreamArgs& a, int h, int slot) {
  return (uint32_t)(h * a.row_head_stride + slot * a.row_slot_stride);
}

// Byte offset in the V LDS tile of 16-byte piece `piece` of token row `tok`:
// rows are 128 B, pieces XOR-swizzled by bits 1..3 of the row index so that
// the 32 rows read by one transposing load spread over all banks.
__device__ __forceinline__ int v_lds_offset(int tok, int piece) {
  return tok * D + 16 * (piece ^ ((tok >> 1) & 7));
}

// Running state of one wave's online softmax over its tokens (row r = lane%16
// of the query group): m2 = running max of the log2-scaled logits, lsum = this
// lane's share of the running exp sum, sigma = running max |V scale| (the P
// operand's reference), acc = O^T tile (d = 16 dblk + 4b + i, query r).
struct WaveState {
  float m2;
  float lsum;
  float sigma;
  float zsum;  // 4-bit format: this lane's share of sum_t p_t * vzero_t
  float corr;  // 4-bit format: this lane's share of sum_t P'_t (the f16 P operand)
  float inv_sigma;  // 1 / sigma (0 while sigma is 0), recomputed only when sigma grows
  f32x4 acc[8];
  __device__ __forceinline__ void reset() {
    m2 = kNegInf;
    lsum = 0.f;
    sigma = 0.f;
    zsum = 0.f;
    corr = 0.f;
    inv_sigma = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // Partial output of the tokens seen so far, o = acc * sigma / l, for d =
  // 16 dblk + 4b + i; returns l (the whole row's exp sum, all lanes).
  __device__ __forceinline__ float finish(f32x4 o[8]) const {
    const float l = wave_sum_xor16_32(lsum);
    const float f = sigma / l;
#pragma unroll
    for (int dblk = 0; dblk < 8; ++dblk) o[dblk] = acc[dblk] * f;
    return l;
  }
  // The same for the 4-bit format.  For the dim pair d = 32 pc + 8b + 2i + (0,
  // 1), with index byte x = n_even + 16 n_odd, acc[2pc] holds sum_t P'_t (1024
  // + x) and acc[2pc + 1] sum_t P'_t (1024 + 16 n_odd).  So o_even = ((acc[2pc]
  // - acc[2pc + 1]) sigma + zsum) / l and o_odd = ((acc[2pc + 1] - 1024 corr)
  // sigma / 16 + zsum) / l; o is returned interleaved, o[2pc + half] = d = 32 pc
  // + 8b + 4 half + 0..3.
  template <int QG>
  __device__ __forceinline__ float finish_tq4(f32x4 o[8]) const {
    // With the compact softmax, lanes r and r + 8 hold the two tiles of query r.
    auto pair = [](float x) { return tq4_compact_softmax(QG) ? x + row_ror8(x) : x; };
    const float l = wave_sum_xor16_32(pair(lsum));
    const float z = wave_sum_xor16_32(pair(zsum));
    const float c1024 = 1024.0f * wave_sum_xor16_32(pair(corr));
    const float f = sigma / l;
    const float f16th = f * 0.0625f;
    const float zl = z / l;
#pragma unroll
    for (int pc = 0; pc < 4; ++pc) {
      const f32x4 e = (acc[2 * pc] - acc[2 * pc + 1]) * f + zl;
      const f32x4 od = (acc[2 * pc + 1] - c1024) * f16th + zl;
      o[2 * pc] = f32x4{e[0], od[0], e[1], od[1]};
      o[2 * pc + 1] = f32x4{e[2], od[2], e[3], od[3]};
    }
    return l;
  }
  template <bool TQ4, int QG>
  __device__ __forceinline__ float finish_as(f32x4 o[8]) const {
    if constexpr (TQ4)
      return finish_tq4<QG>(o);
    else
      return finish(o);
  }
};

// Column of the first of the 4 consecutive dims o[dblk] holds in lane group b,
// as returned by finish (fp8) or finish_tq4 (4-bit format).
template <bool TQ4>
__device__ __forceinline__ int out_col(int dblk, int b) {
  return TQ4 ? 32 * (dblk >> 1) + 8 * b + 4 * (dblk & 1) : 16 * dblk + 4 * b;
}

// Walk tokens [t_begin, t_end) of (s, h) in 32-token chunks, accumulating into
// `w`.  Every `chunks_per_part` chunks, on_boundary(k, w) is called with the
// index k (from 0) of the partition that just ended; it must consume and reset
// `w`.  The caller handles the last partition after the return.  lds_v (8 KiB,
// two stages) and lds_sc (512 B) are this wave's LDS staging area.
template <int QG, int BS, typename OnBoundary>
__device__ __forceinline__ void stream_tokens(const StreamArgs& a, int s, int h, int t_begin,
                                              int t_end, int chunks_per_part, uint8_t* lds_v,
                                              float* lds_sc, WaveState& w,
                                              OnBoundary on_boundary) {
  static_assert(BS == 16 || BS == 32, "kv block size");
  static_assert(QG >= 1 && QG <= 16, "query group size");
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;  // MFMA row/column index within a 16-lane group
  const int b = lane >> 4;  // 16-lane group
  const int Hkv = a.num_kv_heads;
  const int n_chunks = (t_end - t_begin + CHUNK - 1) / CHUNK;
  const int n_blocks = (t_end - t_begin + BS - 1) / BS;  // block-table entries read
  const int32_t* bt_row = a.bt + (size_t)s * a.max_blocks + t_begin / BS;
  const uint32_t nb_max = (uint32_t)a.num_blocks - 1u;

  // Block-table window: lane i holds entry 64*win + i of this range.
  int bt_win = 0;
  int bt_reg = lane < n_blocks ? bt_row[lane] : 0;
  auto block_id = [&](int j) -> uint32_t {  // j: block index within the range, uniform
    if ((j >> 6) != bt_win) {
      bt_win = j >> 6;
      const int e = 64 * bt_win + lane;
      bt_reg = e < n_blocks ? bt_row[e] : 0;
    }
    const uint32_t id = (uint32_t)__builtin_amdgcn_readlane(bt_reg, j & 63);
    return id < nb_max ? id : nb_max;  // negative ids wrap high and clamp too
  };

  // q operand (B of QK^T): lane holds q[row r][32b + 8c .. +7] for c = 0..3.
  bf16x8 qop[4];
  if (r < QG) {
    const uint16_t* qrow = a.q + ((size_t)(s * Hkv + h) * QG + r) * D + 32 * b;
#pragma unroll
    for (int c = 0; c < 4; ++c) qop[c] = *reinterpret_cast<const bf16x8*>(qrow + 8 * c);
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) qop[c] = bf16x8{};
  }

  // Per-lane byte offsets inside a block, fixed for the stream: K pieces of
  // token rows 16t + r (BS 32; row r of either block for BS 16) and V pieces
  // of token rows 8j + lane / 8, in the swizzled piece order.
  const size_t block_bytes = (size_t)Hkv * BS * D;
  uint32_t k_off[2], v_off[4];
#pragma unroll
  for (int t = 0; t < 2; ++t) k_off[t] = row_in_block(a, h, BS == 32 ? 16 * t + r : r) + 32 * b;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tok = 8 * j + (lane >> 3);
    const int piece = (lane & 7) ^ ((tok >> 1) & 7);
    v_off[j] = row_in_block(a, h, BS == 32 ? tok : (tok & 15)) + 16 * piece;
  }

  // Issue the loads of chunk c: K pieces into registers, V rows and scales
  // into LDS stage `st`.
  i32x4 kraw[2][2];
  auto issue = [&](int c, int st) {
    const int jb = (c * CHUNK) / BS;
    const uint32_t blkA = block_id(jb);
    uint32_t blkB = blkA;
    if (BS == 16) blkB = (jb + 1 < n_blocks) ? block_id(jb + 1) : blkA;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t blk = (BS == 32 || t == 0) ? blkA : blkB;
      const uint8_t* src = a.k + (size_t)blk * block_bytes + k_off[t];
      kraw[t][0] = *reinterpret_cast<const i32x4*>(src);
      kraw[t][1] = *reinterpret_cast<const i32x4*>(src + 16);
    }
    uint8_t* vdst = lds_v + st * (CHUNK * D);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t blk = (BS == 32 || j < 2) ? blkA : blkB;  // tokens 16..31: j >= 2
      const uint8_t* src = a.v + (size_t)blk * block_bytes + v_off[j];
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(vdst + 1024 * j), 16, 0,
                                       kCachePolicyStreaming);
    }
    {
      const int field = lane >> 5;
      const int tok = lane & 31;
      const uint32_t blk = (BS == 32 || tok < 16) ? blkA : blkB;
      const int slot = BS == 32 ? tok : (tok & 15);
      const float* src = a.scales + (((size_t)blk * Hkv + h) * 2 + field) * BS + slot;
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(lds_sc + st * (2 * CHUNK)), 4, 0,
                                       kCachePolicyStreaming);
    }
  };

  // Transposing-read address of this lane: MFMA k-slot e of group b is token
  // 16*(e/4) + 4b + e%4 (the order of the QK^T C layout); source lane s of the
  // group supplies k-slot s/2 and column half s%2.
  const int tr_tok = 16 * (r >> 3) + 4 * b + ((r >> 1) & 3);
  const int tr_half = 8 * (r & 1);

  issue(0, 0);
  int next_boundary = chunks_per_part;
  int part_done = 0;
  for (int c = 0; c < n_chunks; ++c) {
    const int st = c & 1;
    // Chunk c's loads are the only ones outstanding: drain them (the LDS
    // writes of global_load_lds complete under vmcnt) and take everything the
    // chunk needs out of LDS before chunk c+1's LDS-direct loads are issued;
    // from then on the chunk is computed from registers only, so no later LDS
    // read has to wait for the in-flight loads.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __builtin_amdgcn_sched_barrier(0);
    const float* sc = lds_sc + st * (2 * CHUNK);
    f32x4 ks0 = *reinterpret_cast<const f32x4*>(sc + 4 * b);
    f32x4 ks1 = *reinterpret_cast<const f32x4*>(sc + 16 + 4 * b);
    f32x4 vs0 = *reinterpret_cast<const f32x4*>(sc + 32 + 4 * b);
    f32x4 vs1 = *reinterpret_cast<const f32x4*>(sc + 48 + 4 * b);
    i32x2 vraw[8];
    const uint8_t* vt = lds_v + st * (CHUNK * D);
#pragma unroll
    for (int dblk = 0; dblk < 8; ++dblk)
      vraw[dblk] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (lds_i32x2*)(vt + v_lds_offset(tr_tok, dblk) + tr_half));
    i32x4 kc[2][2] = {{kraw[0][0], kraw[0][1]}, {kraw[1][0], kraw[1][1]}};
    __builtin_amdgcn_sched_barrier(0);
    if (c + 1 < n_chunks) issue(c + 1, st ^ 1);
    // A partition boundary: its stores go out behind the next chunk's loads.
    if (c == next_boundary) {
      on_boundary(part_done, w);
      ++part_done;
      next_boundary += chunks_per_part;
    }

    const int nvalid = min(CHUNK, t_end - (t_begin + c * CHUNK));

    // ---- QK^T: C[token 4b+i][query r] for tiles 0 and 1 ----
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const int hi = cc >> 1, lo = 2 * (cc & 1);
      const bf16x8 k0 = fp8x8_to_bf16(kc[0][hi][lo], kc[0][hi][lo + 1]);
      const bf16x8 k1 = fp8x8_to_bf16(kc[1][hi][lo], kc[1][hi][lo + 1]);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qop[cc], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qop[cc], s1, 0, 0, 0);
    }

    // ---- scale, mask (this lane's tokens 4b..4b+3 and 16+4b..16+4b+3) ----
    float y[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      y[i] = s0[i] * (ks0[i] * a.qk_scale_log2);
      y[4 + i] = s1[i] * (ks1[i] * a.qk_scale_log2);
    }
    int vmask0 = -1, vmask1 = -1;
    if (nvalid < CHUNK) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool v0 = 4 * b + i < nvalid, v1 = 16 + 4 * b + i < nvalid;
        y[i] = v0 ? y[i] : kNegInf;
        y[4 + i] = v1 ? y[4 + i] : kNegInf;
        vs0[i] = v0 ? vs0[i] : 0.f;
        vs1[i] = v1 ? vs1[i] : 0.f;
        if (!v0) vmask0 &= ~(0xFF << (8 * i));
        if (!v1) vmask1 &= ~(0xFF << (8 * i));
      }
    }

    // ---- online softmax (base 2) ----
    float mx = y[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmax_nn(mx, y[i]);
    mx = wave_max_xor16_32(mx);
    const float m2_new = fmax_nn(w.m2, mx);
    const float alpha = __builtin_amdgcn_exp2f(w.m2 - m2_new);
    float pr[8];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pr[i] = __builtin_amdgcn_exp2f(y[i] - m2_new);
      psum += pr[i];
    }
    w.lsum = w.lsum * alpha + psum;
    w.m2 = m2_new;

    // ---- V-scale reference and P operand ----
    // sigma tracks the largest |V scale|, so |P operand| <= 1 for scales of either sign.
    auto ab = [](float x) { return __builtin_fabsf(x); };
    float vmax = fmax_nn(fmax_nn(fmax_nn(ab(vs0[0]), ab(vs0[1])), fmax_nn(ab(vs0[2]), ab(vs0[3]))),
                         fmax_nn(fmax_nn(ab(vs1[0]), ab(vs1[1])), fmax_nn(ab(vs1[2]), ab(vs1[3]))));
    vmax = wave_max_xor16_32(vmax);
    float acc_scale = alpha;
    if (vmax > w.sigma) {  // uniform: vmax is a wave-wide maximum
      const float inv = 1.0f / vmax;
      acc_scale = alpha * (w.sigma * inv);
      w.sigma = vmax;
      w.inv_sigma = inv;
    }
    const float inv_sigma = w.inv_sigma;
    f16x8 pop;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pop[i] = (_Float16)(pr[i] * (vs0[i] * inv_sigma));
      pop[4 + i] = (_Float16)(pr[4 + i] * (vs1[i] * inv_sigma));
    }
    if (__ballot(acc_scale != 1.0f)) {  // a factor of exactly 1 changes no bits
#pragma unroll
      for (int i = 0; i < 8; ++i) w.acc[i] *= acc_scale;
    }

    // ---- PV: acc[dblk] (O^T[d = 16 dblk + 4b + i][query r]) += V^T P ----
#pragma unroll
    for (int dblk = 0; dblk < 8; ++dblk) {
      const f16x8 vop = fp8x8_to_f16(vraw[dblk][0] & vmask0, vraw[dblk][1] & vmask1);
      w.acc[dblk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pop, w.acc[dblk], 0, 0, 0);
    }
  }
}

// ---------------------------------------------------------------------------
// The 4-bit record format ("TQ" record of the tq_decode page).  A cache block
// is Hkv*BS rows of 128 bytes, head-major [Hkv][BS] or slot-major [BS][Hkv]
// (the page's data region; row_in_block), each with the K indices in bytes
// 0..63 and the V indices in 64..127 (dim d in byte d/2, low nibble for even
// d), then fp16 metadata [Hkv][3][BS]: K norm, V scale, V zero point.
// k = centroids[index] * norm, v = index * scale + zero.
//
// Per-wave LDS of the 4-bit stream: two 4 KiB row stages and two 256 B
// metadata stages ([3][32] fp16), in the same 8.5 KiB staging area as the fp8
// stream's; the centroid table (1 KiB, or 64 KiB per lane in the flat
// kernels) is a workgroup's LDS array of its own.
//  * A chunk's 32 rows of 128 B (a whole block's slots of one kv head when
//    BS = 32, of two blocks when BS = 16) arrive whole, by LDS-direct loads
//    of 8 rows each, and K is read back from LDS.  Splitting each row between a
//    K register load and a V LDS load instead (two requests per 128-byte line)
//    streams about 13 % slower on this GPU.
//  * Row R's 16-byte pieces p = 0..7 (K: 0..3, V: 4..7) sit at slot
//    p ^ tq4_row_swz(R).  The swizzle keeps the K reads (rows 16t + r, piece
//    b) and the transposed V reads (tokens 4b + i and 16 + 4b + i) on distinct
//    16-byte bank groups within every 8 and 16 lanes.
//  * The table is a separate LDS object, one per workgroup, so that the
//    compiler can see that reading it never waits for the row stages'
//    LDS-direct loads.  It maps an index byte to the f16 centroids of its two
//    nibbles, and QK runs on f16 MFMAs with q converted to f16: 11
//    significant bits of the codebook, where bf16's 8 would miss the 1e-2
//    bound on outlier-heavy queries.
constexpr int kTq4RowStage = CHUNK * D;
constexpr int kTq4MetaStage = 256;
constexpr int kTq4MetaOff = 2 * kTq4RowStage;
constexpr int kTq4WaveLds = kTq4MetaOff + 2 * kTq4MetaStage;
constexpr int kTq4TableEntries = 256;
// The per-lane centroid table of the flat kernels: every entry repeated in 64
// adjacent dwords (a 256-byte row), lane l reading the copy in column l, so a
// wave's 64 lookups hit 64 distinct banks whatever the index bytes (random
// bytes otherwise pile several lanes onto one bank: about 30 % of the cycles
// of the flat partition kernel with a one-column table).  A lookup's address,
// index byte n of a dword in bits 8..15 and the lane's column offset in bits
// 0..7, is one byte permute, the same one VALU op as the one-column table's
// shift.  64 KiB: the flat kernels have room for it (one workgroup per CU);
// the kernels of one to eight waves per (s, h) or partition keep one column.
// Tables of 16 or 32 columns in rows of 64 or 128 bytes (not byte aligned)
// took a shift and a mask per lookup and gained less.
constexpr int kTq4LaneCols = 64;
constexpr int tq4_flat_table_cols(bool tq4) { return tq4 ? kTq4LaneCols : 1; }

__device__ __forceinline__ int tq4_row_swz(int row) {
  return (row & 7) ^ ((row >> 3) & 1) ^ ((row >> 2) & 4);
}

// The centroid table, written by threads tid, tid + nthreads, ...: entry x =
// (f16(c[x & 15]), f16(c[x >> 4])), the first in the low half, once (COLS =
// 1) or in each of the 64 columns of row x (COLS = 64).  One table serves
// every wave of a workgroup, at a fixed LDS address, so a lookup's address is
// the index byte times 4 (one shift) plus a constant offset, or with 64
// columns the byte permute described above.
template <int COLS = 1>
__device__ __forceinline__ void build_tq4_table(uint32_t* tab, const float* centroids, int tid,
                                                int nthreads) {
  static_assert(COLS == 1 || COLS == kTq4LaneCols, "table columns");
  if constexpr (COLS == 1) {
    for (int i = tid; i < kTq4TableEntries; i += nthreads) {
      const f16x2 e = {(_Float16)centroids[i & 15], (_Float16)centroids[i >> 4]};
      tab[i] = __builtin_bit_cast(uint32_t, e);
    }
  } else {
    // 16 stores of 4 copies per row.
    u32x4* t4 = reinterpret_cast<u32x4*>(tab);
    for (int i = tid; i < kTq4TableEntries * (COLS / 4); i += nthreads) {
      const int x = i / (COLS / 4);
      const f16x2 e = {(_Float16)centroids[x & 15], (_Float16)centroids[x >> 4]};
      const uint32_t v = __builtin_bit_cast(uint32_t, e);
      t4[i] = u32x4{v, v, v, v};
    }
  }
}

// 8 index bytes x = n_lo + 16 n_hi (one per token) -> f16 operands 1024 + x of
// the whole bytes and 1024 + 16 n_hi of their high nibbles: a byte permute puts
// each byte under the f16 exponent byte 0x64, and a mask clears the low nibble.
// The even dims (low nibbles) follow from the difference of the two
// accumulators; the odd dims from the second less 1024 times the sum of the P
// operand (WaveState::corr), carried at 16x.
__device__ __forceinline__ void tq4_nibbles_f16(i32x2 raw, f16x8& whole, f16x8& hi) {
  constexpr uint32_t kExp = 0x64646464u;
  u32x4 x, h;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    // result bytes: (b0, 0x64, b1, 0x64) and (b2, 0x64, b3, 0x64)
    x[2 * w] = __builtin_amdgcn_perm(kExp, (uint32_t)raw[w], 0x04010400u);
    x[2 * w + 1] = __builtin_amdgcn_perm(kExp, (uint32_t)raw[w], 0x04030402u);
    h[2 * w] = x[2 * w] & 0xFFF0FFF0u;
    h[2 * w + 1] = x[2 * w + 1] & 0xFFF0FFF0u;
  }
  whole = __builtin_bit_cast(f16x8, x);
  hi = __builtin_bit_cast(f16x8, h);
}

template <int V>
struct StageTag {
  static constexpr int value = V;
};

// The 4-bit counterpart of stream_tokens: the same contract and the same
// one-chunk-ahead pipeline.  lds is the wave's staging area (kTq4WaveLds
// bytes); tab the workgroup's centroid table in COLS columns, which build_tq4_table has
// written before any wave streams.
template <int QG, int BS, int COLS, typename OnBoundary>
__device__ __forceinline__ void stream_tokens_tq4(const StreamArgs& a, int s, int h, int t_begin,
                                                  int t_end, int chunks_per_part, uint8_t* lds,
                                                  const uint32_t* tab, WaveState& w,
                                                  OnBoundary on_boundary) {
  static_assert(BS == 16 || BS == 32, "kv block size");
  static_assert(QG >= 1 && QG <= 16, "query group size");
  constexpr bool kCompact = tq4_compact_softmax(QG);
  const int lane = threadIdx.x & 63;
  const uint32_t tab_col = (uint32_t)(lane & (COLS - 1)) << 2;  // byte offset of the lane's column
  static_assert(COLS == 1 || COLS == kTq4LaneCols, "table columns");
  const int r = lane & 15;
  const int b = lane >> 4;
  const int Hkv = a.num_kv_heads;
  const int n_chunks = (t_end - t_begin + CHUNK - 1) / CHUNK;
  const int n_blocks = (t_end - t_begin + BS - 1) / BS;
  const int32_t* bt_row = a.bt + (size_t)s * a.max_blocks + t_begin / BS;
  const uint32_t nb_max = (uint32_t)a.num_blocks - 1u;
  const size_t block_bytes = (size_t)a.tq4_block_bytes;
  const size_t meta_base = (size_t)Hkv * BS * D + (size_t)h * 3 * BS * 2;

  int bt_win = 0;
  int bt_reg = lane < n_blocks ? bt_row[lane] : 0;
  auto block_id = [&](int j) -> uint32_t {
    if ((j >> 6) != bt_win) {
      bt_win = j >> 6;
      const int e = 64 * bt_win + lane;
      bt_reg = e < n_blocks ? bt_row[e] : 0;
    }
    const uint32_t id = (uint32_t)__builtin_amdgcn_readlane(bt_reg, j & 63);
    return id < nb_max ? id : nb_max;
  };

  // q operands in f16, dims 32b + 8c + 0..7 of row r (the d-permutation of
  // stream_tokens).  bf16 -> f16 is exact for magnitudes in [2^-14, 2^15); a
  // group whose largest |q| reaches 2^15 is first scaled by a power of two,
  // 2^-qexp, which the logit scale c2 takes back.
  f16x8 qf[4];
  float c2 = a.qk_scale_log2;
  {
    bf16x8 qop[4];
    if (r < QG) {
      const uint16_t* qrow = a.q + ((size_t)(s * Hkv + h) * QG + r) * D + 32 * b;
#pragma unroll
      for (int c = 0; c < 4; ++c) qop[c] = *reinterpret_cast<const bf16x8*>(qrow + 8 * c);
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) qop[c] = bf16x8{};
    }
    float qmax = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) qmax = fmax_nn(qmax, __builtin_fabsf((float)qop[c][j]));
    qmax = wave_max_all(qmax);
    float qscale = 1.f;
    if (qmax >= 32768.f) {  // uniform
      const int qexp = __builtin_amdgcn_frexp_expf(qmax) - 15;  // qmax * 2^-qexp < 2^15
      qscale = __builtin_ldexpf(1.f, -qexp);
      c2 = __builtin_ldexpf(c2, qexp);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) qf[c][j] = (_Float16)((float)qop[c][j] * qscale);
  }

  // Issue chunk c into LDS stage `st`: its 32 rows, 8 per LDS-direct load
  // (lane l lands at byte 16 l of the load's 1 KiB: row 8j + l/8, slot l % 8,
  // so it fetches piece (l % 8) ^ tq4_row_swz(row)), then the metadata (LDS
  // dword l < 48 = field l / 16, tokens 2 (l % 16) and +1).  Every address is
  // a wave-uniform block base plus a per-lane 32-bit offset fixed for the
  // stream.
  // The loads are buffer loads to LDS: a buffer resource over the block's
  // record (scalar registers) plus a 32-bit lane offset fixed for the stream (a
  // record is below 2^31 bytes), so issuing a chunk takes no vector address
  // arithmetic.
  uint32_t row_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 8 * j + (lane >> 3);
    const int piece = (lane & 7) ^ tq4_row_swz(row);
    const int slot = BS == 32 ? row : (row & 15);
    row_off[j] = row_in_block(a, h, slot) + 16 * piece;
  }
  const int ml = lane < 48 ? lane : 0;
  const uint32_t meta_off =
      (uint32_t)meta_base + (uint32_t)(4 * (BS == 32 ? ml : (ml >> 4) * 8 + (ml & 7)));
  const bool meta_second = BS == 16 && (ml & 15) >= 8;  // tokens 16..31: the second block
  auto issue = [&](int c, int st) {
    const int jb = (c * CHUNK) / BS;
    const uint32_t blkA = block_id(jb);
    uint32_t blkB = blkA;
    if (BS == 16) blkB = (jb + 1 < n_blocks) ? block_id(jb + 1) : blkA;
    const __amdgpu_buffer_rsrc_t recA = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.tq4) + (size_t)blkA * block_bytes, 0, (int)block_bytes, kBufferDword3);
    const __amdgpu_buffer_rsrc_t recB = BS == 32 ? recA : __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.tq4) + (size_t)blkB * block_bytes, 0, (int)block_bytes, kBufferDword3);
    uint8_t* rdst = lds + st * kTq4RowStage;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds((BS == 32 || j < 2) ? recA : recB,
                                               (lds_void*)(rdst + 1024 * j), 16, row_off[j], 0, 0,
                                               kCachePolicyStreaming);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(meta_second ? recB : recA,
                                             (lds_void*)(lds + kTq4MetaOff + st * kTq4MetaStage), 4,
                                             meta_off, 0, 0, kCachePolicyStreaming);
  };

  const int tr_tok = 16 * (r >> 3) + 4 * b + ((r >> 1) & 3);
  const int tr_half = 8 * (r & 1);
  const int tr_swz = tq4_row_swz(tr_tok);

  issue(0, 0);
  int next_boundary = chunks_per_part;
  int part_done = 0;
  // Lane (r, b)'s K pieces: row 16 t + r, piece b.
  const int k_slot = b ^ tq4_row_swz(r);
  // One chunk; the stage is a compile-time constant (the loop below is unrolled
  // by two), so every stage address is a fixed offset from a loop-invariant
  // base.
  auto step = [&](int c, auto stage) {
    constexpr int st = decltype(stage)::value;
    // Chunk c has landed in stage st.  Its stage reads are issued first: an
    // LDS read of the staging area after the next chunk's LDS-direct loads
    // would wait for them.  Then chunk c + 1 goes to stage st ^ 1 (last read
    // for chunk c - 1, whose values have all been used), and the centroid
    // lookups, which read only the table, follow.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* rows = lds + st * kTq4RowStage;
    i32x4 kraw[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
      kraw[t] = *reinterpret_cast<const i32x4*>(rows + (16 * t + r) * D + 16 * (k_slot ^ (4 * t)));
    const uint8_t* meta = lds + kTq4MetaOff + st * kTq4MetaStage;
    // Metadata of this lane's tokens: 4b + i and 16 + 4b + i, or with the
    // compact softmax only tile r / 8 (see below).
    f16x4 kn0, kn1, vs0h, vs1h, vz0h, vz1h;
    if constexpr (kCompact) {
      const int mo = 2 * (16 * (r >> 3) + 4 * b);
      kn0 = *reinterpret_cast<const f16x4*>(meta + mo);
      vs0h = *reinterpret_cast<const f16x4*>(meta + 64 + mo);
      vz0h = *reinterpret_cast<const f16x4*>(meta + 128 + mo);
    } else {
      kn0 = *reinterpret_cast<const f16x4*>(meta + 2 * (4 * b));
      kn1 = *reinterpret_cast<const f16x4*>(meta + 2 * (16 + 4 * b));
      vs0h = *reinterpret_cast<const f16x4*>(meta + 64 + 2 * (4 * b));
      vs1h = *reinterpret_cast<const f16x4*>(meta + 64 + 2 * (16 + 4 * b));
      vz0h = *reinterpret_cast<const f16x4*>(meta + 128 + 2 * (4 * b));
      vz1h = *reinterpret_cast<const f16x4*>(meta + 128 + 2 * (16 + 4 * b));
    }
    i32x2 vraw[4];
#pragma unroll
    for (int pc = 0; pc < 4; ++pc)
      vraw[pc] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (lds_i32x2*)(rows + tr_tok * D + 16 * ((4 + pc) ^ tr_swz) + tr_half));
    __builtin_amdgcn_sched_barrier(0);
    if (c + 1 < n_chunks) issue(c + 1, st ^ 1);
    __builtin_amdgcn_sched_barrier(0);
    // K operands: kop[t][cc] = the centroids of the 4 index bytes of dword cc,
    // dims 8cc + 0..7.
    f16x8 kop[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const uint32_t x = (uint32_t)kraw[t][cc];
        if constexpr (COLS == 1) {
          kop[t][cc] = __builtin_bit_cast(
              f16x8, u32x4{tab[x & 0xFF], tab[(x >> 8) & 0xFF], tab[(x >> 16) & 0xFF], tab[x >> 24]});
        } else {
          // Entry e's row starts at byte 256 e: v_perm_b32 puts index byte n of
          // x in bits 8..15 and the lane's column offset (bits 0..7 of tab_col)
          // below it.
          const char* tb = reinterpret_cast<const char*>(tab);
          auto at = [&](uint32_t sel) {
            return *reinterpret_cast<const uint32_t*>(tb + __builtin_amdgcn_perm(x, tab_col, sel));
          };
          kop[t][cc] = __builtin_bit_cast(
              f16x8, u32x4{at(0x0C0C0400u), at(0x0C0C0500u), at(0x0C0C0600u), at(0x0C0C0700u)});
        }
      }
    if (c == next_boundary) {
      on_boundary(part_done, w);
      ++part_done;
      next_boundary += chunks_per_part;
    }

    const int nvalid = min(CHUNK, t_end - (t_begin + c * CHUNK));

    // ---- QK^T: C[token 4b+i][query r] for tiles 0 and 1 ----
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[0][k], qf[k], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[1][k], qf[k], s1, 0, 0, 0);
    }

    // ---- softmax and P operand ----
    f16x8 pop;
    if constexpr (kCompact) {
      // QG <= 8 uses only query columns r < 8, so lanes r >= 8 take over tile
      // 1 of query r - 8 (the MFMA's results moved by 8 lanes within each row):
      // each lane then handles 4 tokens, 16 (r / 8) + 4b + i, instead of 8.
      // The max reductions add one step across the two halves of a row; the
      // sums are paired up the same way at the end (finish_tq4).  The P
      // operand of lane r < 8 is its own 4 values followed by lane r + 8's.
      float y[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sc = __int_as_float(__builtin_amdgcn_update_dpp(
            __float_as_int(s0[i]), __float_as_int(s1[i]), 0x118, 0xF, 0xC, false));  // row_shr:8
        y[i] = __builtin_fmaf((float)kn0[i], sc, 0.f);
      }
      f16x4 vs = vs0h, vz = vz0h;
      if (nvalid < CHUNK) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool v = 16 * (r >> 3) + 4 * b + i < nvalid;
          y[i] = v ? y[i] : kNegInf;
          vs[i] = v ? vs[i] : (_Float16)0;
          vz[i] = v ? vz[i] : (_Float16)0;
        }
      }
      float mx = fmax_nn(fmax_nn(y[0], y[1]), fmax_nn(y[2], y[3]));
      mx = fmax_nn(mx, row_ror8(mx));
      mx = wave_max_xor16_32(mx);
      const float m2_new = fmax_nn(w.m2, mx * c2);  // c2 > 0: the max commutes with it
      const float alpha = __builtin_amdgcn_exp2f(w.m2 - m2_new);
      float pr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(y[i], c2, -m2_new));
      const float psum = (pr[0] + pr[1]) + (pr[2] + pr[3]);
      float zs = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) zs = __builtin_fmaf((float)vz[i], pr[i], zs);
      w.lsum = w.lsum * alpha + psum;
      w.zsum = w.zsum * alpha + zs;
      w.m2 = m2_new;

      auto ab = [](_Float16 x) { return __builtin_fabsf((float)x); };  // sigma: largest |V scale|
      float vmax = fmax_nn(fmax_nn(ab(vs[0]), ab(vs[1])), fmax_nn(ab(vs[2]), ab(vs[3])));
      vmax = fmax_nn(vmax, row_ror8(vmax));
      vmax = wave_max_xor16_32(vmax);
      float acc_scale = alpha;
      if (vmax > w.sigma) {  // uniform: vmax is a wave-wide maximum
        const float inv = 1.0f / vmax;
        acc_scale = alpha * (w.sigma * inv);
        w.sigma = vmax;
        w.inv_sigma = inv;
      }
      const float inv_sigma = w.inv_sigma;
      const f16x2 own01 = {(_Float16)(pr[0] * __builtin_fmaf((float)vs[0], inv_sigma, 0.f)),
                           (_Float16)(pr[1] * __builtin_fmaf((float)vs[1], inv_sigma, 0.f))};
      const f16x2 own23 = {(_Float16)(pr[2] * __builtin_fmaf((float)vs[2], inv_sigma, 0.f)),
                           (_Float16)(pr[3] * __builtin_fmaf((float)vs[3], inv_sigma, 0.f))};
      const int o01 = __builtin_bit_cast(int, own01), o23 = __builtin_bit_cast(int, own23);
      const int t01 = __builtin_amdgcn_update_dpp(0, o01, 0x128, 0xF, 0xF, false);  // row_ror:8
      const int t23 = __builtin_amdgcn_update_dpp(0, o23, 0x128, 0xF, 0xF, false);
      pop = __builtin_bit_cast(f16x8, i32x4{o01, o23, t01, t23});
      if (__ballot(acc_scale != 1.0f)) {  // a factor of exactly 1 changes no bits
#pragma unroll
        for (int i = 0; i < 8; ++i) w.acc[i] *= acc_scale;
        w.corr *= acc_scale;
      }
      // corr += this lane's own 4 P' values; lane r + 8's are added at the end
      const f16x2 one = {(_Float16)1, (_Float16)1};
      w.corr = __builtin_amdgcn_fdot2(own23, one, __builtin_amdgcn_fdot2(own01, one, w.corr, false),
                                      false);
    } else {
      // ---- logits y = s * kn, mask ----
      // y is the base-2 logit divided by qk_scale_log2: the factor enters with
      // the exponent, exp2(y c - m2), one fused multiply-add.  The fp16 K norm,
      // V scale and V zero point enter their products through mixed-precision
      // fused multiply-adds, with no separate conversion.
      float y[8];
  #pragma unroll
      for (int i = 0; i < 4; ++i) {
        y[i] = __builtin_fmaf((float)kn0[i], s0[i], 0.f);
        y[4 + i] = __builtin_fmaf((float)kn1[i], s1[i], 0.f);
      }
      f16x4 vs0 = vs0h, vs1 = vs1h, vz0 = vz0h, vz1 = vz1h;
      if (nvalid < CHUNK) {
  #pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool v0 = 4 * b + i < nvalid, v1 = 16 + 4 * b + i < nvalid;
          y[i] = v0 ? y[i] : kNegInf;
          y[4 + i] = v1 ? y[4 + i] : kNegInf;
          vs0[i] = v0 ? vs0[i] : (_Float16)0;
          vs1[i] = v1 ? vs1[i] : (_Float16)0;
          vz0[i] = v0 ? vz0[i] : (_Float16)0;
          vz1[i] = v1 ? vz1[i] : (_Float16)0;
        }
      }

      // ---- online softmax (base 2) ----
      float mx = y[0];
  #pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmax_nn(mx, y[i]);
      mx = wave_max_xor16_32(mx);
      const float m2_new = fmax_nn(w.m2, mx * c2);  // c2 > 0: the max commutes with it
      const float alpha = __builtin_amdgcn_exp2f(w.m2 - m2_new);
      float pr[8];
      float psum = 0.f, zs = 0.f;
  #pragma unroll
      for (int i = 0; i < 8; ++i) {
        pr[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(y[i], c2, -m2_new));
        psum += pr[i];
      }
  #pragma unroll
      for (int i = 0; i < 4; ++i) zs = __builtin_fmaf((float)vz0[i], pr[i], zs);
  #pragma unroll
      for (int i = 0; i < 4; ++i) zs = __builtin_fmaf((float)vz1[i], pr[4 + i], zs);
      w.lsum = w.lsum * alpha + psum;
      w.zsum = w.zsum * alpha + zs;
      w.m2 = m2_new;

      // ---- V-scale reference and P operand ----
      // sigma: the largest |V scale|
      const f16x4 vsm = __builtin_elementwise_max(__builtin_elementwise_abs(vs0),
                                                  __builtin_elementwise_abs(vs1));
      float vmax = fmax_nn(fmax_nn((float)vsm[0], (float)vsm[1]), fmax_nn((float)vsm[2], (float)vsm[3]));
      vmax = wave_max_xor16_32(vmax);
      float acc_scale = alpha;
      if (vmax > w.sigma) {  // uniform: vmax is a wave-wide maximum
        const float inv = 1.0f / vmax;
        acc_scale = alpha * (w.sigma * inv);
        w.sigma = vmax;
        w.inv_sigma = inv;
      }
      const float inv_sigma = w.inv_sigma;
  #pragma unroll
      for (int i = 0; i < 4; ++i) {
        pop[i] = (_Float16)(pr[i] * __builtin_fmaf((float)vs0[i], inv_sigma, 0.f));
        pop[4 + i] = (_Float16)(pr[4 + i] * __builtin_fmaf((float)vs1[i], inv_sigma, 0.f));
      }
      if (__ballot(acc_scale != 1.0f)) {  // a factor of exactly 1 changes no bits
  #pragma unroll
        for (int i = 0; i < 8; ++i) w.acc[i] *= acc_scale;
        w.corr *= acc_scale;
      }
      {  // corr += sum of this lane's 8 P' values, exactly as the MFMA sees them
        const f16x2 one = {(_Float16)1, (_Float16)1};
        float c = w.corr;
  #pragma unroll
        for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_fdot2(f16x2{pop[2 * i], pop[2 * i + 1]}, one, c, false);
        w.corr = c;
      }
    }

    // ---- PV: acc[2pc], acc[2pc + 1] (dim pair 32 pc + 2m, m = 4b + i) += V^T P ----
#pragma unroll
    for (int pc = 0; pc < 4; ++pc) {
      f16x8 vwhole, vhi;
      tq4_nibbles_f16(vraw[pc], vwhole, vhi);
      w.acc[2 * pc] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vwhole, pop, w.acc[2 * pc], 0, 0, 0);
      w.acc[2 * pc + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vhi, pop, w.acc[2 * pc + 1], 0, 0, 0);
    }
  };
  for (int c = 0; c < n_chunks; c += 2) {
    step(c, StageTag<0>{});
    if (c + 1 < n_chunks) step(c + 1, StageTag<1>{});
  }
}

// One stream call for either format (lds_v: the wave's staging area, lds_sc:
// the fp8 scale stages inside it, lds_tab: the wave's 4-bit centroid table).
template <int QG, int BS, bool TQ4, int COLS = 1, typename OnBoundary>
__device__ __forceinline__ void stream_any(const StreamArgs& a, int s, int h, int t_begin, int t_end,
                                           int chunks_per_part, uint8_t* lds_v, float* lds_sc,
                                           const uint32_t* lds_tab, WaveState& w,
                                           OnBoundary on_boundary) {
  if constexpr (TQ4)
    stream_tokens_tq4<QG, BS, COLS>(a, s, h, t_begin, t_end, chunks_per_part, lds_v, lds_tab, w,
                              on_boundary);
  else
    stream_tokens<QG, BS>(a, s, h, t_begin, t_end, chunks_per_part, lds_v, lds_sc, w, on_boundary);
}

// Clamp a device-side sequence length into [0, cap].
__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

// Per-wave LDS staging area: for fp8, two 4 KiB V stages + two 256 B scale
// stages; for 4-bit, two 4 KiB row stages + two 256 B metadata stages.  After
// the stream the same bytes hold the wave's normalised partial (up to 16 rows
// x 512 B) and its max logits / exp sums (2 x 16 floats).
constexpr int kWaveLds = 2 * CHUNK * D + 2 * 2 * CHUNK * 4;
static_assert(kTq4WaveLds <= kWaveLds, "4-bit staging area");
static_assert(16 * D * 4 + 2 * 16 * 4 <= kWaveLds, "merge area must fit the staging area");

// Partial triple of partition p of (s, h) = sh: o_p = acc * sigma / l_p, m_p
// (natural log units), l_p, rows r < QG; then the running state restarts.
// With a.nt_partials (a uniform branch) o_p goes out through buffer stores
// that carry the non-temporal bit: a plain store and a non-temporal one in the
// two arms of a branch would be merged into one plain store by the compiler.
template <int QG, bool TQ4>
__device__ __forceinline__ void store_partial(const PartitionArgs& a, int sh, int p, WaveState& w) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, b = lane >> 4;
  f32x4 o[8];
  const float l = w.template finish_as<TQ4, QG>(o);
  const size_t block = ((size_t)sh * a.num_partitions + p) * QG;  // the partition's first row
  if (a.nt_partials) {
    // The partition's QG x 128 floats as one buffer with a wave-uniform base.
    const uint64_t base = reinterpret_cast<uint64_t>(a.o + block * D);
    float* base_u = reinterpret_cast<float*>(
        ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(base >> 32)) << 32) |
        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)base));
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(base_u, 0, QG * D * 4, kBufferDword3);
    if (r < QG) {
#pragma unroll
      for (int dblk = 0; dblk < 8; ++dblk)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o[dblk]), rs,
                                               (r * D + out_col<TQ4>(dblk, b)) * 4, 0,
                                               kCachePolicyStreaming);
    }
  } else if (r < QG) {
    float* dst = a.o + (block + r) * D;
#pragma unroll
    for (int dblk = 0; dblk < 8; ++dblk)
      *reinterpret_cast<f32x4*>(dst + out_col<TQ4>(dblk, b)) = o[dblk];
  }
  if (r < QG && b == 0) {
    a.ml[block + r] = w.m2 * kLn2;
    a.es[block + r] = l;
  }
  w.reset();
}

// Split-K partition kernel: one wave per group of `parts_per_wave`
// consecutive partitions of one (s, h); writes the partial triple of every
// live partition in the group (STEP G).
template <int QG, int BS, bool TQ4>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void tq_partition_kernel(PartitionArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_stage[kWaveLds];
  __shared__ __attribute__((aligned(16))) uint32_t lds_tab[TQ4 ? kTq4TableEntries : 1];
  const int lane = threadIdx.x;
  const int P = a.num_partitions;
  const int Hkv = a.st.num_kv_heads;
  const int E = a.partition_tokens;
  const int ppw = a.parts_per_wave;
  // The partition groups of one (s, h) are consecutive workgroups, which keeps
  // its partial stores together (an order with (s, h) fastest scattered them
  // and lost 8 % on the bandwidth workload); with a.rotate their order is
  // rotated by sh, so that group p of every (s, h) does not land on one XCD
  // (rotate_units says when).
  const int n_groups = (P + ppw - 1) / ppw;
  const int sh = blockIdx.x / n_groups;
  const int pg = a.rotate ? (int)((blockIdx.x % n_groups + (unsigned)sh) % (unsigned)n_groups)
                          : (int)(blockIdx.x % n_groups);
  const int h = sh % Hkv;
  const int s = sh / Hkv;
  const int p0 = pg * ppw;
  const int L = clamp_len(a.seq_lens[s], a.len_cap);
  const int t_begin = p0 * E;
  if (t_begin >= L) return;  // dead partitions: nothing is written
  const int t_end = min(t_begin + min(ppw, P - p0) * E, L);
  if constexpr (TQ4) build_tq4_table(lds_tab, a.st.centroids, lane, 64);

  WaveState w;
  w.reset();
  const int chunks_per_part = E / CHUNK;
  stream_any<QG, BS, TQ4>(a.st, s, h, t_begin, t_end, chunks_per_part, lds_stage,
                          reinterpret_cast<float*>(lds_stage + 2 * CHUNK * D), lds_tab, w,
                          [&](int k, WaveState& ws) { store_partial<QG, TQ4>(a, sh, p0 + k, ws); });
  const int n_chunks = (t_end - t_begin + CHUNK - 1) / CHUNK;
  store_partial<QG, TQ4>(a, sh, p0 + (n_chunks - 1) / chunks_per_part, w);
}


// Log-sum-exp merge of n partials j = 0..n-1 for 4 columns, in j order:
// o = sum_j (l_j e^{m_j - M} / sum_j' l_j' e^{m_j' - M}) o_j.  ld_o(j) returns
// the 4 columns of o_j, ld_m(j) / ld_l(j) its max logit and exp sum.  Returns
// the merged exp sum and max through *l_out, *m_out.  A single partial is
// returned as is.
template <typename LdO, typename LdM, typename LdL>
__device__ __forceinline__ f32x4 lse_merge4(int n, LdO ld_o, LdM ld_m, LdL ld_l, float* m_out,
                                            float* l_out) {
  if (n == 1) {
    *m_out = ld_m(0);
    *l_out = ld_l(0);
    return ld_o(0);
  }
  float M = kNegInf;
  for (int j = 0; j < n; ++j) M = fmaxf(M, ld_m(j));
  float Wsum = 0.f;
  for (int j = 0; j < n; ++j) Wsum += ld_l(j) * __expf(ld_m(j) - M);
  const float invW = 1.0f / Wsum;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < n; ++j) {
    const float wt = ld_l(j) * __expf(ld_m(j) - M) * invW;
    o += wt * ld_o(j);
  }
  *m_out = M;
  *l_out = Wsum;
  return o;
}

// Log-sum-exp merge of n <= NMAX partials (the formula of lse_merge4) with
// every load issued up front, so the loads take one round trip.
template <int NMAX, typename LdO, typename LdM, typename LdL>
__device__ __forceinline__ f32x4 lse_merge4_regs(int n, LdO ld_o, LdM ld_m, LdL ld_l,
                                                 float* m_out = nullptr, float* l_out = nullptr) {
  if (n == 1) {  // a single partial is returned as is
    if (m_out) *m_out = ld_m(0);
    if (l_out) *l_out = ld_l(0);
    return ld_o(0);
  }
  float mj[NMAX], lj[NMAX];
  f32x4 oj[NMAX];
#pragma unroll
  for (int j = 0; j < NMAX; ++j) {
    if (j < n) {
      mj[j] = ld_m(j);
      lj[j] = ld_l(j);
      oj[j] = ld_o(j);
    }
  }
  float M = kNegInf;
#pragma unroll
  for (int j = 0; j < NMAX; ++j)
    if (j < n) M = fmaxf(M, mj[j]);
  float Wsum = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NMAX; ++j) {
    if (j < n) {
      const float wt = lj[j] * __expf(mj[j] - M);
      Wsum += wt;
      o += wt * oj[j];
    }
  }
  if (m_out) *m_out = M;
  if (l_out) *l_out = Wsum;
  return o * (1.0f / Wsum);
}

// Device-coherent loads and stores of the cross-workgroup partials: buffer
// accesses with the sc1 cache policy, what an agent-scope relaxed atomic
// access is on gfx940-family devices.  They write through to, and read from,
// the point where all XCDs see the same bytes, so no L2-wide write-back or
// invalidate is needed around them; unlike atomics they move 16 bytes at a
// time and the compiler may keep many in flight.  A buffer resource covers one
// workspace array (wave-uniform base); offsets are 32-bit byte offsets.
constexpr int kCachePolicyAgent = 16;  // sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const float* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, (int)bytes, kBufferDword3);
}
__device__ __forceinline__ void st_coherent4(__amdgpu_buffer_rsrc_t rs, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, off, 0, kCachePolicyAgent);
}
__device__ __forceinline__ void st_coherent1(__amdgpu_buffer_rsrc_t rs, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs, off, 0, kCachePolicyAgent);
}
__device__ __forceinline__ f32x4 ld_coherent4(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kCachePolicyAgent));
}
__device__ __forceinline__ float ld_coherent1(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, kCachePolicyAgent));
}

// The release half of the cross-workgroup exchange: wait until every store
// this thread issued has completed (vmcnt = 0; the sc1 stores are then visible
// to all XCDs), before the barrier that precedes the arrival count.  Written as
// inline assembly with a memory clobber, so that the compiler may not move any
// memory access across it (the s_waitcnt builtin alone does not touch memory
// in the compiler's model, so a store could be scheduled after it).  The
// order store -> s_waitcnt vmcnt(0) -> s_barrier -> atomic add is checked in
// the built assembly by a CPU test.
__device__ __forceinline__ void drain_stores_release() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__device__ __forceinline__ void store_bf16x4(uint16_t* dst, f32x4 o) {
  const uint32_t lo = (uint32_t)f32_to_bf16_rne(o[0]) | ((uint32_t)f32_to_bf16_rne(o[1]) << 16);
  const uint32_t hi = (uint32_t)f32_to_bf16_rne(o[2]) | ((uint32_t)f32_to_bf16_rne(o[3]) << 16);
  *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
}

// Fused decode.  Each (s, h) gets `splits` workgroups of W waves; its tile
// groups (256 tokens) are dealt in contiguous runs to the workgroups, and
// within a workgroup to its waves.  Each wave keeps one online softmax over
// its run; the workgroup merges its waves' partials by log-sum-exp through
// LDS.  With one workgroup of work for the (s, h), that merge writes bf16 out.
// Otherwise each workgroup writes its merged partial (o, m, l) to the
// workspace, releases it at device scope and counts itself in; the last to
// arrive acquires all partials, merges them in workgroup order (so the result
// does not depend on arrival order), writes out and re-arms the counter to 0.
template <int QG, int BS, bool TQ4>
__global__ __launch_bounds__(512) void tq_fused_kernel(FusedArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
  __shared__ __attribute__((aligned(16))) uint32_t lds_tab[TQ4 ? kTq4TableEntries : 1];
  __shared__ int last_arrival;
  if constexpr (TQ4) {  // before any return: every thread reaches the barrier
    build_tq4_table(lds_tab, a.st.centroids, threadIdx.x, blockDim.x);
    __syncthreads();
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  const int r = lane & 15;
  const int b = lane >> 4;
  const int Hkv = a.st.num_kv_heads;
  const int splits = a.splits;
  // The workgroups of one (s, h) are consecutive; with a.rotate their split
  // order is rotated by sh, as in tq_partition_kernel.
  const int sh = blockIdx.x / splits;
  const int split = a.rotate ? (int)((blockIdx.x % splits + (unsigned)sh) % (unsigned)splits)
                             : (int)(blockIdx.x % splits);
  const int h = sh % Hkv;
  const int s = sh / Hkv;
  const int L = clamp_len(a.seq_lens[s], a.len_cap);
  uint16_t* out = a.out + (size_t)sh * QG * D;
  if (L == 0) {  // uniform over the workgroup
    if (split == 0)
      for (int idx = threadIdx.x; idx < QG * (D / 4); idx += blockDim.x)
        *reinterpret_cast<uint2*>(out + 4 * idx) = make_uint2(0u, 0u);
    return;
  }
  constexpr int TG = kTokensPerTileGroup;
  const int n_tg = (L + TG - 1) / TG;
  const int per_wg = (n_tg + splits - 1) / splits;
  const int n_wg = (n_tg + per_wg - 1) / per_wg;  // workgroups of this (s, h) with work
  if (split >= n_wg) return;                        // no work, does not count itself in
  const int tg0 = split * per_wg;
  const int cnt = min(per_wg, n_tg - tg0);
  const int per_wave = (cnt + W - 1) / W;
  const int n_used = (cnt + per_wave - 1) / per_wave;

  uint8_t* region = lds_dyn + wave * kWaveLds;
  float* part_o = reinterpret_cast<float*>(region);               // [QG][128]
  float* part_m = reinterpret_cast<float*>(region + 16 * D * 4);  // [QG]
  float* part_l = part_m + 16;                                    // [QG]
  if (wave < n_used) {  // uniform over the wave
    const int t_begin = (tg0 + wave * per_wave) * TG;
    const int t_end = min(t_begin + per_wave * TG, min((tg0 + cnt) * TG, L));
    WaveState w;
    w.reset();
    stream_any<QG, BS, TQ4>(a.st, s, h, t_begin, t_end, 0x7fffffff, region,
                            reinterpret_cast<float*>(region + 2 * CHUNK * D),
                            lds_tab, w,
                            [](int, WaveState&) {});
    f32x4 o[8];
    const float l = w.template finish_as<TQ4, QG>(o);
    if (r < QG) {
#pragma unroll
      for (int dblk = 0; dblk < 8; ++dblk)
        *reinterpret_cast<f32x4*>(part_o + r * D + out_col<TQ4>(dblk, b)) = o[dblk];
      if (b == 0) {
        part_m[r] = w.m2 * kLn2;
        part_l[r] = l;
      }
    }
  }
  __syncthreads();

  // Merge this workgroup's waves.
  const float* lds_f = reinterpret_cast<const float*>(lds_dyn);
  constexpr int kWaveF = kWaveLds / 4;
  const uint32_t wsrow0 = ((uint32_t)sh * splits + split) * QG;
  const size_t ws_rows = (size_t)gridDim.x * QG;  // [S*Hkv][splits][QG]
  const __amdgpu_buffer_rsrc_t rs_o = coherent_rsrc(a.ws_o, ws_rows * D * 4);
  const __amdgpu_buffer_rsrc_t rs_m = coherent_rsrc(a.ws_m, ws_rows * 4);
  const __amdgpu_buffer_rsrc_t rs_l = coherent_rsrc(a.ws_l, ws_rows * 4);
  for (int idx = threadIdx.x; idx < QG * (D / 4); idx += blockDim.x) {
    const int g = idx / (D / 4);
    const int col = 4 * (idx % (D / 4));
    float m, l;
    const f32x4 o = lse_merge4(
        n_used,
        [&](int v) { return *reinterpret_cast<const f32x4*>(lds_f + v * kWaveF + g * D + col); },
        [&](int v) { return lds_f[v * kWaveF + 16 * D + g]; },
        [&](int v) { return lds_f[v * kWaveF + 16 * D + 16 + g]; }, &m, &l);
    if (n_wg == 1) {
      store_bf16x4(out + g * D + col, o);
    } else {
      st_coherent4(rs_o, ((wsrow0 + g) * D + col) * 4, o);
      if (col == 0) {
        st_coherent1(rs_m, (wsrow0 + g) * 4, m);
        st_coherent1(rs_l, (wsrow0 + g) * 4, l);
      }
    }
  }
  if (n_wg == 1) return;

  // Cross-workgroup merge.  Release: every thread's coherent stores complete
  // (vmcnt drained) before the barrier, and only then is the arrival counted.
  // Acquire: the last arrival reads the partials with coherent loads issued
  // after its count returned.
  drain_stores_release();
  __syncthreads();
  if (threadIdx.x == 0)
    last_arrival = __hip_atomic_fetch_add(a.counters + sh, 1, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT) == n_wg - 1;
  __syncthreads();
  if (!last_arrival) return;
  if (threadIdx.x == 0)  // re-arm for the next call; every arrival of this launch is in
    __hip_atomic_store(a.counters + sh, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // At most kFusedMaxSplits partials: every load of the merge in flight at once.
  const uint32_t row_sh = (uint32_t)sh * splits * QG;
  for (int idx = threadIdx.x; idx < QG * (D / 4); idx += blockDim.x) {
    const int g = idx / (D / 4);
    const int col = 4 * (idx % (D / 4));
    const f32x4 o = lse_merge4_regs<kFusedMaxSplits>(
        n_wg, [&](int j) { return ld_coherent4(rs_o, ((row_sh + j * QG + g) * D + col) * 4); },
        [&](int j) { return ld_coherent1(rs_m, (row_sh + j * QG + g) * 4); },
        [&](int j) { return ld_coherent1(rs_l, (row_sh + j * QG + g) * 4); });
    store_bf16x4(out + g * D + col, o);
  }
}

// Fused decode over a flat work list, dealt evenly.  The live 32-token chunks
// (kFlatUnitTokens) of all (s, h) form one list in (s, h, chunk) order, T
// entries long.  The grid's G workgroups of W waves hold N = G*W waves, of
// which the first Nu = min(N, T) take consecutive ranges of q = T / Nu
// entries, the first T % Nu of them one more: every wave streams the same
// number of chunks, to within one, however ragged the lengths are.  (With
// whole tile groups as entries, long-context batches of a few tile groups per
// wave left half the waves one tile group longer than the rest.)  Workgroup g holds
// the waves g*W .. g*W+W-1.
// A wave's range is cut into segments at (s, h) boundaries; each segment gets
// one online softmax.  A segment that holds a whole (s, h) is finished by its
// wave, which writes bf16 out.  Any other segment is a piece: only a wave's
// first or last segment can be one.  The wave stores a piece's partial (o, m,
// l) in LDS: the last piece in its staging area, free once the stream is done;
// the first in a slot of its own (fp8) or, for the 4-bit format, held in
// registers until the stream is done (FlatLayout).  After a barrier the workgroup merges
// the pieces of each (s, h) it holds, in wave order.  If the (s, h) lies
// inside the workgroup's range, that merge writes out.  Otherwise (only the
// workgroup's first or last (s, h) can reach outside) the merged partial goes
// to workspace slot 2g (the workgroup's first (s, h)) or 2g+1 (its last),
// released at device scope, and the workgroup counts itself in on the (s, h)'s
// counter; the last arrival merges the partials of workgroups g_first ..
// g_last in workgroup order (so the result does not depend on arrival order),
// writes out and re-arms the counter to 0.  The list and all its indices
// follow from the device-side lengths and the grid alone.  Zero-length
// sequences are not in the list: workgroup g zeroes the rows of sequences g,
// g+G, ... that have none.

// Inclusive prefix sum over the 64 lanes of a wave by DPP: shifts by 1, 2, 4, 8
// within each 16-lane row, then row 0's and row 2's last lane added to rows 1
// and 3 (row_bcast:15) and lane 31 added to rows 2 and 3 (row_bcast:31).
// Lanes whose source is outside the row, or whose row is masked off, add 0.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}


template <int QG, bool TQ4>
struct FlatLayout {
  // A partial in LDS or the workspace: o [QG][128], then m [16] and l [16].
  static constexpr int kPieceFloats = QG * D + 32;
  static constexpr int kPieceBytes = kPieceFloats * 4;
  static_assert(kPieceBytes <= kWaveLds, "the last piece must fit the staging area");
  // fp8: per-wave LDS is the staging area (which also holds the last piece),
  // then the first piece, stored when its segment ends.  4-bit: the per-lane
  // centroid table takes 64 KiB, so a wave keeps its first piece in registers
  // until its stream is done and then stores it behind the last piece in its
  // staging area (QG <= 8), or, where the two do not fit (QG = 16), in the
  // table's LDS once every wave of the workgroup is past its lookups.
  static constexpr bool kFirstInRegs = TQ4;
  static constexpr bool kFirstInStage = TQ4 && 2 * kPieceBytes <= kWaveLds;
  static constexpr bool kFirstInTable = TQ4 && !kFirstInStage;
  static constexpr int kArea = TQ4 ? kWaveLds : kWaveLds + kPieceBytes;  // per wave, dynamic
  // The table's LDS array, in dwords (it also holds the first pieces when kFirstInTable).
  static constexpr int kTableWords =
      !TQ4 ? 1
           : (kFirstInTable && kFlatWaves * kPieceFloats > kTq4TableEntries * kTq4LaneCols
                  ? kFlatWaves * kPieceFloats
                  : kTq4TableEntries * kTq4LaneCols);
  // Byte offset of wave v's first piece: in the dynamic area, or (kFirstInTable) in the table array.
  static constexpr int first_offset(int v) {
    return kFirstInTable ? v * kPieceBytes : v * kArea + (TQ4 ? kPieceBytes : kWaveLds);
  }
};

// Store the wave's finished partial (rows r < QG) at piece P.
template <int QG, bool TQ4>
__device__ __forceinline__ void store_piece(float* P, const f32x4 o[8], float m, float l) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, b = lane >> 4;
  if (r < QG) {
#pragma unroll
    for (int dblk = 0; dblk < 8; ++dblk)
      *reinterpret_cast<f32x4*>(P + r * D + out_col<TQ4>(dblk, b)) = o[dblk];
    if (b == 0) {
      P[QG * D + r] = m;
      P[QG * D + 16 + r] = l;
    }
  }
}

template <int QG, int BS, bool TQ4>
__global__ __launch_bounds__(64 * kFlatWaves) void tq_flat_kernel(FlatArgs a) {
  using Lay = FlatLayout<QG, TQ4>;
  constexpr int kTabCols = tq4_flat_table_cols(TQ4);
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
  __shared__ __attribute__((aligned(16))) uint32_t lds_tab[Lay::kTableWords];
  __shared__ int piece_sh[2 * kFlatWaves];        // s*Hkv+h of wave v's first (2v) / last
                                                  // (2v+1) piece, -1: none
  __shared__ int piece_ea[2 * kFlatWaves];        // list offset of that (s, h)'s first entry
  __shared__ int piece_n[2 * kFlatWaves];         // its entries
  __shared__ int arrived_last[2];
  constexpr int TG = kFlatUnitTokens;  // tokens per list entry, a power of two
  constexpr int ush = __builtin_ctz(TG);
  static_assert(TG == 1 << ush && TG % CHUNK == 0, "list entries are whole chunks");
  constexpr int kItems = QG * (D / 4);  // (row, 4 columns) items of one merge, <= blockDim
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  const int S = a.num_seqs;
  const int Hkv = a.st.num_kv_heads;
  const int G = gridDim.x;
  const int g = blockIdx.x;
  auto len_of = [&](int s) { return clamp_len(a.seq_lens[s], a.len_cap); };
  if constexpr (TQ4) {  // before any return: every thread reaches the barrier
    build_tq4_table<kTabCols>(lds_tab, a.st.centroids, threadIdx.x, blockDim.x);
    __syncthreads();
  }

  // List entries per kv head, per wave in registers: lane l holds the clamped
  // lengths of sequences s = l + 64 i (i < k <= kFlatSlices); per slice i an inclusive
  // scan over the lanes gives the list offsets within the slice.
  const int k = (S + 63) >> 6;
  int len_r[kFlatSlices], incl_r[kFlatSlices], slice_total[kFlatSlices];
  int total = 0;
  // All loads first (in bounds; slices past k skipped by uniform branches), so
  // they share one wait.
#pragma unroll
  for (int i = 0; i < kFlatSlices; ++i)
    len_r[i] = i < k ? a.seq_lens[min(lane + 64 * i, S - 1)] : 0;
#pragma unroll
  for (int i = 0; i < kFlatSlices; ++i) {
    len_r[i] = (i < k && lane + 64 * i < S) ? clamp_len(len_r[i], a.len_cap) : 0;
    incl_r[i] = 0;
    slice_total[i] = 0;
    if (i < k) {
      incl_r[i] = wave_inclusive_scan((len_r[i] + TG - 1) >> ush);
      slice_total[i] = __builtin_amdgcn_readlane(incl_r[i], 63);
      total += slice_total[i];
    }
  }
  const int T = total * Hkv;

  // Zero the rows of empty sequences g, g + G, ...
  for (int s = g; s < S; s += G) {
    int Ls = 0;
#pragma unroll
    for (int i = 0; i < kFlatSlices; ++i)
      if (i == (s >> 6)) Ls = __builtin_amdgcn_readlane(len_r[i], s & 63);
    if (Ls == 0) {
      uint16_t* o = a.out + (size_t)s * Hkv * QG * D;
      for (int idx = threadIdx.x; idx < Hkv * QG * (D / 4); idx += blockDim.x)
        *reinterpret_cast<uint2*>(o + 4 * idx) = make_uint2(0u, 0u);
    }
  }

  // Nu = min(N, T) waves in use; wave x takes q or q + 1 entries: the first
  // `rem` waves one more.
  const int Nw = G * W;
  const int Nu = T < Nw ? T : Nw;
  const int gw0 = g * W;
  if (gw0 >= Nu) return;  // uniform over the workgroup (T = 0 included)
  const int Wu = Nu - gw0 < W ? Nu - gw0 : W;
  const int q = T / Nu, rem = T - q * Nu;
  auto entry_of = [&](int x) { return x * q + (x < rem ? x : rem); };  // first entry of wave x
  auto wave_of = [&](int e) {                                           // wave holding entry e
    const int big = rem * (q + 1);
    return e < big ? e / (q + 1) : rem + (e - big) / q;
  };
  const int wg_begin = entry_of(gw0);
  const int wg_end = entry_of(gw0 + Wu);
  const int gw = gw0 + (wave < Wu ? wave : Wu - 1);
  const int A = entry_of(gw);
  const int B = entry_of(gw + 1);
  // Locate entry A: its slice, then the first lane of the slice whose
  // sequences reach past it.  base = list offset of (s, h = 0).
  int s = S - 1, L = 0, n = 0, base = 0;
  {
    int sb = 0;
#pragma unroll
    for (int i = 0; i < kFlatSlices; ++i) {
      if (i < k && A >= sb * Hkv && A < (sb + slice_total[i]) * Hkv) {
        const int ln = __builtin_ctzll(__ballot((sb + incl_r[i]) * Hkv > A));
        L = __builtin_amdgcn_readlane(len_r[i], ln);
        n = (L + TG - 1) >> ush;
        s = 64 * i + ln;
        base = (sb + __builtin_amdgcn_readlane(incl_r[i], ln) - n) * Hkv;
      }
      sb += slice_total[i];
    }
  }

  uint8_t* area = lds_dyn + wave * Lay::kArea;
  float* last_piece = reinterpret_cast<float*>(area);
  uint8_t* const first_base = Lay::kFirstInTable ? reinterpret_cast<uint8_t*>(lds_tab) : lds_dyn;
  float* first_piece = reinterpret_cast<float*>(first_base + Lay::first_offset(wave));
  int f_sh = -1, l_sh = -1, f_n = 0, l_n = 0;
  int f_ea = 0, l_ea = 0;
  f32x4 f_o[Lay::kFirstInRegs ? 8 : 1];  // the first piece while the stream goes on
  float f_m = 0.f, f_l = 0.f;
  if (wave < Wu) {  // uniform over the wave
    int h = n > 0 ? (A - base) / n : Hkv;
    int k0 = n > 0 ? (A - base) - h * n : 0;
    int pos = A;
    bool first_seg = true;
    while (h < Hkv) {  // h >= Hkv only if the lengths changed under the kernel
      const int k1 = min(n, k0 + (B - pos));
      const int sh = s * Hkv + h;
      WaveState st;
      st.reset();
      stream_any<QG, BS, TQ4, kTabCols>(a.st, s, h, k0 * TG, min(k1 * TG, L), 0x7fffffff, area,
                              reinterpret_cast<float*>(area + 2 * CHUNK * D),
                              lds_tab, st,
                              [](int, WaveState&) {});
      f32x4 o[8];
      const float l = st.template finish_as<TQ4, QG>(o);
      if (k0 == 0 && k1 == n) {  // the whole (s, h)
        const int r = lane & 15, b = lane >> 4;
        if (r < QG) {
          uint16_t* dst = a.out + ((size_t)sh * QG + r) * D;
#pragma unroll
          for (int dblk = 0; dblk < 8; ++dblk) store_bf16x4(dst + out_col<TQ4>(dblk, b), o[dblk]);
        }
      } else if (first_seg) {
        if constexpr (Lay::kFirstInRegs) {
#pragma unroll
          for (int dblk = 0; dblk < 8; ++dblk) f_o[dblk] = o[dblk];
          f_m = st.m2 * kLn2;
          f_l = l;
        } else {
          store_piece<QG, TQ4>(first_piece, o, st.m2 * kLn2, l);
        }
        f_sh = sh;
        f_ea = base + h * n;
        f_n = n;
      } else {  // a piece that is not the first is the wave's last segment
        store_piece<QG, TQ4>(last_piece, o, st.m2 * kLn2, l);
        l_sh = sh;
        l_ea = base + h * n;
        l_n = n;
      }
      pos += k1 - k0;
      if (pos >= B) break;
      // Next (s, h) of the list: the next kv head, or the next non-empty sequence.
      first_seg = false;
      k0 = 0;
      if (++h == Hkv) {
        h = 0;
        base += n * Hkv;
        do {
          if (++s >= S) {
            h = Hkv;
            break;
          }
          L = len_of(s);
          n = (L + TG - 1) >> ush;
        } while (n == 0);
      }
    }
  }
  if constexpr (Lay::kFirstInStage)
    if (f_sh >= 0) store_piece<QG, TQ4>(first_piece, f_o, f_m, f_l);
  if (lane == 0) {
    piece_sh[2 * wave] = f_sh;
    piece_ea[2 * wave] = f_ea;
    piece_n[2 * wave] = f_n;
    piece_sh[2 * wave + 1] = l_sh;
    piece_ea[2 * wave + 1] = l_ea;
    piece_n[2 * wave + 1] = l_n;
  }
  __syncthreads();
  if constexpr (Lay::kFirstInTable) {  // every wave is past its lookups
    if (f_sh >= 0) store_piece<QG, TQ4>(first_piece, f_o, f_m, f_l);
    __syncthreads();
  }

  // Merge the pieces of each (s, h) this workgroup holds.  Piece p = 2v + which
  // is wave v's first (which = 0) or last piece.  The pieces of one (s, h) are
  // consecutive: piece p0 = 2v0 + w0, then the first pieces of waves v0+1 ..
  // v1.  Every wave finds the runs alike, lane p reading piece p.  At most two
  // of these (s, h) reach outside the workgroup.
  auto piece = [&](int v, int which) -> const float* {
    return reinterpret_cast<const float*>(which == 0 ? first_base + Lay::first_offset(v)
                                                     : lds_dyn + v * Lay::kArea);
  };
  const int t = threadIdx.x;
  const int item_g = t / (D / 4);
  const int item_col = 4 * (t % (D / 4));
  const size_t ws_rows = (size_t)2 * G * QG;  // the workspace's partial rows
  const __amdgpu_buffer_rsrc_t rs_o = coherent_rsrc(a.ws_o, ws_rows * D * 4);
  const __amdgpu_buffer_rsrc_t rs_m = coherent_rsrc(a.ws_m, ws_rows * 4);
  const __amdgpu_buffer_rsrc_t rs_l = coherent_rsrc(a.ws_l, ws_rows * 4);
  int ext_sh[2] = {-1, -1};
  int ext_ea[2] = {0, 0};
  int ext_n[2] = {0, 0};
  // A wave's last piece always begins a run; its first piece continues the
  // previous wave's last one exactly when the (s, h) began before the wave's
  // range (piece_ea < the wave's first entry), except in the first wave.
  const int my_sh = lane < 2 * Wu ? piece_sh[lane] : -1;
  const int my_ea = lane < 2 * Wu ? piece_ea[lane] : 0;
  const int my_n = lane < 2 * Wu ? piece_n[lane] : 0;
  const bool cont = (lane & 1) == 0 && lane > 0 && my_ea < entry_of(gw0 + (lane >> 1));
  const uint64_t have = __ballot(my_sh >= 0);
  uint64_t starts = __ballot(my_sh >= 0 && !cont);
  while (starts) {
    const int p0 = __builtin_ctzll(starts);
    starts &= starts - 1;
    const uint64_t before_next = starts ? (1ull << __builtin_ctzll(starts)) - 1 : ~0ull;
    const int p1 = 63 - __builtin_clzll(have & before_next);
    const int v = p0 >> 1, which = p0 & 1, v1 = p1 >> 1;
    const int sh = __builtin_amdgcn_readlane(my_sh, p0);
    const int ea = __builtin_amdgcn_readlane(my_ea, p0);
    const int n = __builtin_amdgcn_readlane(my_n, p0);
    const bool inside = ea >= wg_begin && ea + n <= wg_end;
    const int slot = ea <= wg_begin ? 0 : 1;
    if (t < kItems) {
      // Piece j of the run: p0's area for j = 0, else wave v + j's first piece.
      const float* first = piece(v, which);
      auto at = [&](int j) { return j == 0 ? first : piece(v + j, 0); };
      float m, l;
      const f32x4 o = lse_merge4_regs<kFlatWaves>(
          v1 - v + 1,
          [&](int j) { return *reinterpret_cast<const f32x4*>(at(j) + item_g * D + item_col); },
          [&](int j) { return at(j)[QG * D + item_g]; },
          [&](int j) { return at(j)[QG * D + 16 + item_g]; }, &m, &l);
      if (inside) {
        store_bf16x4(a.out + ((size_t)sh * QG + item_g) * D + item_col, o);
      } else {
        const uint32_t row = (2 * (uint32_t)g + slot) * QG + item_g;
        st_coherent4(rs_o, (row * D + item_col) * 4, o);
        if (item_col == 0) {
          st_coherent1(rs_m, row * 4, m);
          st_coherent1(rs_l, row * 4, l);
        }
      }
    }
    if (!inside) {
      ext_sh[slot] = sh;
      ext_ea[slot] = ea;
      ext_n[slot] = n;
    }
  }
  if (ext_sh[0] < 0 && ext_sh[1] < 0) return;

  // Release: every thread's coherent stores complete before the barrier, and
  // only then does the workgroup count itself in.
  drain_stores_release();
  __syncthreads();
  int count[2] = {0, 0}, g_first[2] = {0, 0}, first_slot[2] = {0, 0};
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    if (ext_sh[x] < 0) continue;
    const int ea = ext_ea[x], eb = ea + ext_n[x];
    // The waves holding its first and last entries, clamped into the grid so
    // that lengths changed under the kernel cannot index past the workspace.
    const int wf = min(max(wave_of(ea), 0), Nu - 1);
    const int wl = min(max(wave_of(eb - 1), 0), Nu - 1);
    g_first[x] = wf / W;
    count[x] = max(wl / W - g_first[x] + 1, 0);
    first_slot[x] = entry_of(g_first[x] * W) == ea ? 0 : 1;
    if (t == 0)
      arrived_last[x] = __hip_atomic_fetch_add(a.counters + ext_sh[x], 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT) == count[x] - 1;
  }
  __syncthreads();
  // The last arrival merges the n partials of workgroups g_first .. g_first +
  // n - 1 in workgroup order.  With at most kFlatFewPartials of them, every
  // item thread loads the max logits, exp sums and its 4 columns of all of
  // them at once (one round trip) and merges them as lse_merge4_regs does.
  // Otherwise, first the coefficients c_j = l_j e^{m_j - M} / sum_j' l_j'
  // e^{m_j' - M} of each query row, one row per wave at a time, the lanes
  // over j (n <= G <= 256), into LDS (the staging areas are free by now); then
  // every item thread sums c_j o_j for its 4 columns, eight partials' loads in
  // flight at once.
  constexpr int kFlatFewPartials = 8;
  float* coef = reinterpret_cast<float*>(lds_dyn);  // [QG][n]
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    if (ext_sh[x] < 0 || !arrived_last[x]) continue;  // uniform over the workgroup
    if (t == 0)  // re-arm for the next call; every workgroup of this launch is in
      __hip_atomic_store(a.counters + ext_sh[x], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int n = count[x], gf = g_first[x], fs = first_slot[x];
    auto rec = [&](int j) -> uint32_t { return 2 * (uint32_t)(gf + j) + (j == 0 ? fs : 0); };
    if (n <= kFlatFewPartials) {  // uniform over the workgroup
      if (t < kItems) {
        const f32x4 o = lse_merge4_regs<kFlatFewPartials>(
            n, [&](int j) { return ld_coherent4(rs_o, ((rec(j) * QG + item_g) * D + item_col) * 4); },
            [&](int j) { return ld_coherent1(rs_m, (rec(j) * QG + item_g) * 4); },
            [&](int j) { return ld_coherent1(rs_l, (rec(j) * QG + item_g) * 4); });
        store_bf16x4(a.out + ((size_t)ext_sh[x] * QG + item_g) * D + item_col, o);
      }
      continue;
    }
    for (int g = wave; g < QG; g += W) {
      float mj[kFlatGroupsPerLane], lj[kFlatGroupsPerLane];
#pragma unroll
      for (int i = 0; i < kFlatGroupsPerLane; ++i) {
        const int j = lane + 64 * i;
        const bool valid = j < n;
        mj[i] = valid ? ld_coherent1(rs_m, (rec(j) * QG + g) * 4) : kNegInf;
        lj[i] = valid ? ld_coherent1(rs_l, (rec(j) * QG + g) * 4) : 0.f;
      }
      float M = mj[0];
#pragma unroll
      for (int i = 1; i < kFlatGroupsPerLane; ++i) M = fmax_nn(M, mj[i]);
      M = wave_max_all(M);
      float e[kFlatGroupsPerLane], sum = 0.f;
#pragma unroll
      for (int i = 0; i < kFlatGroupsPerLane; ++i) {
        e[i] = lj[i] * __expf(mj[i] - M);
        sum += e[i];
      }
      const float inv = 1.0f / wave_sum_all(sum);
#pragma unroll
      for (int i = 0; i < kFlatGroupsPerLane; ++i)
        if (lane + 64 * i < n) coef[g * n + lane + 64 * i] = e[i] * inv;
    }
    __syncthreads();
    if (t < kItems) {
      f32x4 o = {0.f, 0.f, 0.f, 0.f};
      for (int j0 = 0; j0 < n; j0 += 8) {
        f32x4 oj[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          oj[u] = j0 + u < n ? ld_coherent4(rs_o, ((rec(j0 + u) * QG + item_g) * D + item_col) * 4)
                             : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (j0 + u < n) o += coef[item_g * n + j0 + u] * oj[u];
      }
      store_bf16x4(a.out + ((size_t)ext_sh[x] * QG + item_g) * D + item_col, o);
    }
    __syncthreads();  // the coefficients are read before x + 1 overwrites them
  }
}

// Split-K partition kernel over one flat work list: the live partitions of
// every (s, h) in (s, h, p) order, dealt evenly to the waves of n_groups
// workgroups of kFlatWaves waves (one resident round), as tq_flat_kernel deals
// its chunks.  A wave's run is cut at (s, h) boundaries; each piece is one
// stream whose partials are written at every partition end (STEP G), so the
// partials are bit for bit those of tq_partition_kernel.  No merge and no
// barrier after the set-up: a wave with nothing to do returns.  Used for the
// 4-bit format, whose per-partition waves would each build the centroid
// table and fill the pipeline for only 8 chunks.
template <int QG, int BS, bool TQ4>
__global__ __launch_bounds__(64 * kFlatWaves) void tq_partition_flat_kernel(PartitionArgs a) {
  constexpr int kTabCols = tq4_flat_table_cols(TQ4);
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
  __shared__ __attribute__((aligned(16))) uint32_t lds_tab[TQ4 ? kTq4TableEntries * kTabCols : 1];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  const int S = a.num_seqs;
  const int Hkv = a.st.num_kv_heads;
  const int E = a.partition_tokens;
  auto len_of = [&](int s) { return clamp_len(a.seq_lens[s], a.len_cap); };
  if constexpr (TQ4) {  // before any return: every thread reaches the barrier
    build_tq4_table<kTabCols>(lds_tab, a.st.centroids, threadIdx.x, blockDim.x);
    __syncthreads();
  }

  // Live partitions per kv head: lane l holds the clamped lengths of sequences
  // s = l + 64 i (i < k <= kFlatSlices); per slice an inclusive scan over the
  // lanes gives the list offsets within the slice.
  const int k = (S + 63) >> 6;
  int len_r[kFlatSlices], incl_r[kFlatSlices], slice_total[kFlatSlices];
  int total = 0;
#pragma unroll
  for (int i = 0; i < kFlatSlices; ++i)
    len_r[i] = i < k ? a.seq_lens[min(lane + 64 * i, S - 1)] : 0;
#pragma unroll
  for (int i = 0; i < kFlatSlices; ++i) {
    len_r[i] = (i < k && lane + 64 * i < S) ? clamp_len(len_r[i], a.len_cap) : 0;
    incl_r[i] = 0;
    slice_total[i] = 0;
    if (i < k) {
      incl_r[i] = wave_inclusive_scan((len_r[i] + E - 1) / E);
      slice_total[i] = __builtin_amdgcn_readlane(incl_r[i], 63);
      total += slice_total[i];
    }
  }
  const int T = total * Hkv;

  // Nu = min(waves, T) waves in use; wave x takes q or q + 1 entries, the first
  // `rem` waves one more.
  const int Nw = gridDim.x * W;
  const int Nu = T < Nw ? T : Nw;
  const int gw = blockIdx.x * W + wave;
  if (gw >= Nu) return;
  const int q = T / Nu, rem = T - q * Nu;
  const int A = gw * q + (gw < rem ? gw : rem);
  const int B = A + q + (gw < rem ? 1 : 0);
  // Locate entry A: its slice, then the first lane of the slice whose
  // sequences reach past it.  base = list offset of (s, h = 0).
  int s = S - 1, L = 0, n = 0, base = 0;
  {
    int sb = 0;
#pragma unroll
    for (int i = 0; i < kFlatSlices; ++i) {
      if (i < k && A >= sb * Hkv && A < (sb + slice_total[i]) * Hkv) {
        const int ln = __builtin_ctzll(__ballot((sb + incl_r[i]) * Hkv > A));
        L = __builtin_amdgcn_readlane(len_r[i], ln);
        n = (L + E - 1) / E;
        s = 64 * i + ln;
        base = (sb + __builtin_amdgcn_readlane(incl_r[i], ln) - n) * Hkv;
      }
      sb += slice_total[i];
    }
  }

  uint8_t* area = lds_dyn + wave * kWaveLds;
  const int chunks_per_part = E / CHUNK;
  int h = n > 0 ? (A - base) / n : Hkv;
  int k0 = n > 0 ? (A - base) - h * n : 0;
  int pos = A;
  while (h < Hkv) {  // h >= Hkv only if the lengths changed under the kernel
    const int k1 = min(n, k0 + (B - pos));
    const int sh = s * Hkv + h;
    const int t_begin = k0 * E, t_end = min(k1 * E, L);
    WaveState w;
    w.reset();
    stream_any<QG, BS, TQ4, kTabCols>(a.st, s, h, t_begin, t_end, chunks_per_part, area,
                                      reinterpret_cast<float*>(area + 2 * CHUNK * D), lds_tab, w,
                                      [&](int j, WaveState& ws) { store_partial<QG, TQ4>(a, sh, k0 + j, ws); });
    const int n_chunks = (t_end - t_begin + CHUNK - 1) / CHUNK;
    store_partial<QG, TQ4>(a, sh, k0 + (n_chunks - 1) / chunks_per_part, w);
    pos += k1 - k0;
    if (pos >= B) break;
    // Next (s, h) of the list: the next kv head, or the next non-empty sequence.
    k0 = 0;
    if (++h == Hkv) {
      h = 0;
      do {
        if (++s >= S) {
          h = Hkv;
          break;
        }
        L = len_of(s);
        n = (L + E - 1) / E;
      } while (n == 0);
    }
  }
}

// Merge of the split-K partials: one 256-thread block per (sequence, kv
// head).  Each wave takes query rows g = wave, wave + 4, ...; its lanes read
// the live partitions' max logits and exp sums, reduce M = max m_p and
// W = sum l_p e^{m_p - M} across the wave, and store the coefficients
// c[g][p] = l_p e^{m_p - M} / W in LDS.  Then every thread accumulates
// sum_p c[g][p] o_p for 4 columns of one row with independent 16-byte loads.
// One live partition is copied (c = 1).  More than kMergeMaxParts live
// partitions fall back to recomputing the coefficients per thread.
constexpr int kMergeMaxParts = 256;

__global__ __launch_bounds__(256) void tq_merge_kernel(ReduceArgs a) {
  __shared__ float coef[16 * kMergeMaxParts];
  const int sh = blockIdx.x;
  const int QG = a.query_group_size;
  const int P = a.num_partitions;
  const int s = sh / a.num_kv_heads;
  const int L = clamp_len(a.seq_lens[s], a.len_cap);
  const int live = (L + a.partition_tokens - 1) / a.partition_tokens;  // <= P (host-validated)
  const size_t row_sh = (size_t)sh * P * QG;  // (s, h, p = 0, g = 0)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool staged = live > 1 && live <= kMergeMaxParts;
  if (staged) {
    for (int g = wave; g < QG; g += 4) {
      float mx = kNegInf;
      for (int p = lane; p < live; p += 64) mx = fmaxf(mx, a.ml[row_sh + (size_t)p * QG + g]);
      for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
      float wsum = 0.f;
      for (int p = lane; p < live; p += 64) {
        const size_t rp = row_sh + (size_t)p * QG + g;
        const float w = a.es[rp] * __expf(a.ml[rp] - mx);
        coef[g * kMergeMaxParts + p] = w;
        wsum += w;
      }
      for (int off = 32; off > 0; off >>= 1) wsum += __shfl_xor(wsum, off, 64);
      const float inv = 1.0f / wsum;
      for (int p = lane; p < live; p += 64) coef[g * kMergeMaxParts + p] *= inv;
    }
    __syncthreads();
  }
  for (int idx = threadIdx.x; idx < QG * (D / 4); idx += blockDim.x) {
    const int g = idx / (D / 4);
    const int col = 4 * (idx % (D / 4));
    uint16_t* dst = a.out + ((size_t)sh * QG + g) * D + col;
    const float* src = a.o + (row_sh + g) * D + col;  // partition p at + p * QG * D
    const size_t pstride = (size_t)QG * D;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    if (live == 1) {
      o = *reinterpret_cast<const f32x4*>(src);
    } else if (staged) {
      // 8 independent loads in flight per thread, summed in a fixed order.
      const float* c = coef + g * kMergeMaxParts;
      f32x4 acc[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      int p = 0;
      for (; p + 8 <= live; p += 8) {
        f32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const f32x4*>(src + (p + u) * pstride);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[u] += c[p + u] * v[u];
      }
      for (int u = 0; p < live; ++p, ++u) acc[u] += c[p] * *reinterpret_cast<const f32x4*>(src + p * pstride);
      o = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
    } else if (live > 1) {
      float m, l;
      o = lse_merge4(
          live, [&](int p) { return *reinterpret_cast<const f32x4*>(src + p * pstride); },
          [&](int p) { return a.ml[row_sh + (size_t)p * QG + g]; },
          [&](int p) { return a.es[row_sh + (size_t)p * QG + g]; }, &m, &l);
    }
    store_bf16x4(dst, o);
  }
}

// KV-cache writer: 8 lanes per (new token t, kv head h) row, 8 rows per wave
// (32 per 256-thread workgroup); lane j of a row holds dims 16j .. 16j+15 of
// its K row and of its V row, loaded as two 16-byte pieces each, so a wave
// reads 2 KiB of each contiguous input.  Each row is quantized on its own: s
// = absmax / 448 (absmax over the row's 8 lanes), codes = e4m3fn(x / s) (IEEE
// fp32 division, round to nearest even, clamped to +-448 so the convert never
// overflows), all-zero rows get s = 0 and codes 0.  A row's 128 codes go out as
// one 16-byte store per lane, a whole 128-byte line; lanes 0 and 1 of the row
// write the K and V scales.  A slot outside [0, NB*BS) is skipped (negative:
// padding by convention).
constexpr int kKvRowsPerWg = 32;

__global__ __launch_bounds__(256) void tq_kv_write_kernel(KvWriteArgs a) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 7;
  const int64_t row = (int64_t)blockIdx.x * kKvRowsPerWg + (threadIdx.x >> 3);  // (t, h)
  // A row's 8 lanes are alike in every branch below, and every cross-lane
  // step stays within them.
  if (row >= (int64_t)a.num_tokens * a.num_kv_heads) return;
  const int Hkv = a.num_kv_heads;
  const int t = (int)(row / Hkv);
  const int h = (int)(row % Hkv);
  const int slot = a.slot_mapping[t];
  if (slot < 0 || slot >= a.num_slots) return;
  const int BS = a.kv_block_size;
  const int blk = slot / BS;
  const int off = slot % BS;
  const size_t src = (size_t)row * D + 16 * j;  // bf16 elements
  const size_t dst = (size_t)blk * Hkv * BS * D +
                     (uint32_t)(h * a.row_head_stride + off * a.row_slot_stride) + 16 * j;  // bytes
  u32x4 in[2][2];
#pragma unroll
  for (int field = 0; field < 2; ++field) {
    const u32x4* p = reinterpret_cast<const u32x4*>((field == 0 ? a.k_new : a.v_new) + src);
    in[field][0] = p[0];
    in[field][1] = p[1];
  }
#pragma unroll
  for (int field = 0; field < 2; ++field) {
    float x[16];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const uint32_t pair = in[field][w >> 2][w & 3];
      x[2 * w] = __uint_as_float(pair << 16);
      x[2 * w + 1] = __uint_as_float(pair & 0xffff0000u);
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
    for (int o = 4; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    const float scale = amax / 448.0f;
    u32x4 codes = {0u, 0u, 0u, 0u};
    if (scale > 0.f) {
      // The quotients x / scale, rounded as an IEEE division rounds them, with
      // one division per row: for y = RN(1 / scale), q0 = RN(x y) is within
      // an ulp of x / scale, the residual x - q0 scale is exact in one fused
      // multiply-add, and RN(q0 + r y) is the correctly rounded quotient
      // (Markstein's theorem), given no underflow or overflow in these steps:
      // scale in [2^-90, FLT_MAX] (quotients that could reach an fp8 code are
      // then normal, and so are their residuals).  Zero quotients take the
      // sign of x, as the division's do.  Other rows divide.
      const bool one_div = scale >= 0x1p-90f && scale <= __FLT_MAX__;
      const float y = 1.0f / scale;
      auto quot = [&](float v) {
        if (!one_div) return v / scale;
        const float q0 = v * y;
        const float r = __builtin_fmaf(-q0, scale, v);
        return __builtin_copysignf(__builtin_fmaf(r, y, q0), v);
      };
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float q0 = fminf(fmaxf(quot(x[4 * w]), -448.0f), 448.0f);
        const float q1 = fminf(fmaxf(quot(x[4 * w + 1]), -448.0f), 448.0f);
        const float q2 = fminf(fmaxf(quot(x[4 * w + 2]), -448.0f), 448.0f);
        const float q3 = fminf(fmaxf(quot(x[4 * w + 3]), -448.0f), 448.0f);
        int c = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
        c = __builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, c, true);
        codes[w] = (uint32_t)c;
      }
    }
    *reinterpret_cast<u32x4*>((field == 0 ? a.k : a.v) + dst) = codes;
    if (j == field) a.scales[(((size_t)blk * Hkv + h) * 2 + field) * BS + off] = scale;
  }
}

// The TQ_VALIDATE debug check (see ValidateArgs).  Reads only: lengths are
// clamped into [0, max_seq_len] before they size the block walk, so every
// block-table read stays inside the caller's [S][max_blocks] table.
__global__ __launch_bounds__(64) void tq_validate_kernel(ValidateArgs a) {
  const int s = blockIdx.x;
  const int lane = threadIdx.x;
  const int L = a.seq_lens[s];
  if (lane == 0 && (L < 0 || L > a.max_seq_len))
    printf("tq_validate: seq_lens[%d] = %d is outside [0, %d]\n", s, L, a.max_seq_len);
  const int Lc = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
  const int n = (Lc + a.kv_block_size - 1) / a.kv_block_size;
  const int32_t* row = a.bt + (size_t)s * a.max_blocks;
  for (int j0 = 0; j0 < n; j0 += 64) {
    const int j = j0 + lane;
    const int id = j < n ? row[j] : 0;
    const uint64_t bad = __ballot(j < n && (id < 0 || id >= a.num_blocks));
    if (bad) {
      const int first = __builtin_ctzll(bad);
      if (lane == first)
        printf("tq_validate: block_tables[%d][%d] = %d is outside [0, %d) (token %d < seq_lens %d)\n",
               s, j, id, a.num_blocks, j * a.kv_block_size, Lc);
      break;  // one report per sequence; uniform over the wave
    }
  }
}

// Zero n16 16-byte words at p (a grid-stride loop, every access below n16).
__global__ __launch_bounds__(256) void tq_zero_fill_kernel(u32x4* p, uint32_t n16) {
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < n16; i += gridDim.x * 256u)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

}  // namespace

int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static int cus[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();  // must not surface as a later launch's status
    return kFlatGroupsMax;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) {
      (void)hipGetLastError();
      n = kFlatGroupsMax;
    }
    cus[dev] = n;
  }
  return cus[dev];
}

hipError_t static_scratch(void** ptr, hipStream_t stream) {
  // One device address per GPU, taken once with that GPU current; the first
  // call on a GPU also enqueues the zero fill of its copy on `stream`, ahead
  // of the caller's kernel (the counters must start at zero; every call
  // leaves them at zero again).
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* dev_ptr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!dev_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    static_assert(kStaticScratchBytes % 16 == 0 && kStaticScratchBytes / 16 < (size_t(1) << 32),
                  "scratch size");
    hipLaunchKernelGGL(tq_zero_fill_kernel, dim3(256), dim3(256), 0, stream, static_cast<u32x4*>(p),
                       (uint32_t)(kStaticScratchBytes / 16));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    dev_ptr[dev] = p;
  }
  *ptr = dev_ptr[dev];
  return hipSuccess;
}

// Run LAUNCH_T<QG, BS, TQ4>(args...) for the runtime sizes and format.
#define TQ_DISPATCH(LAUNCH_T, qg, bs, tq4, ...)                                              \
  do {                                                                                      \
    if ((qg) == 6 && (bs) == 16) return (tq4) ? LAUNCH_T<6, 16, true>(__VA_ARGS__)           \
                                              : LAUNCH_T<6, 16, false>(__VA_ARGS__);        \
    if ((qg) == 6 && (bs) == 32) return (tq4) ? LAUNCH_T<6, 32, true>(__VA_ARGS__)           \
                                              : LAUNCH_T<6, 32, false>(__VA_ARGS__);        \
    if ((qg) == 8 && (bs) == 16) return (tq4) ? LAUNCH_T<8, 16, true>(__VA_ARGS__)           \
                                              : LAUNCH_T<8, 16, false>(__VA_ARGS__);        \
    if ((qg) == 8 && (bs) == 32) return (tq4) ? LAUNCH_T<8, 32, true>(__VA_ARGS__)           \
                                              : LAUNCH_T<8, 32, false>(__VA_ARGS__);        \
    if ((qg) == 16 && (bs) == 16) return (tq4) ? LAUNCH_T<16, 16, true>(__VA_ARGS__)         \
                                               : LAUNCH_T<16, 16, false>(__VA_ARGS__);      \
    if ((qg) == 16 && (bs) == 32) return (tq4) ? LAUNCH_T<16, 32, true>(__VA_ARGS__)         \
                                               : LAUNCH_T<16, 32, false>(__VA_ARGS__);      \
    return hipErrorInvalidValue;                                                            \
  } while (0)

template <int QG, int BS, bool TQ4>
hipError_t launch_flat_t(const FlatArgs& a, hipStream_t stream) {
  constexpr size_t lds = (size_t)kFlatWaves * FlatLayout<QG, TQ4>::kArea;
  static_assert(lds + FlatLayout<QG, TQ4>::kTableWords * 4 + 1024 <= 160 * 1024,
                "LDS per workgroup");
  // Dynamic LDS beyond 64 KiB needs the opt-in, once; an error here only means
  // the runtime needs none, and must not leak into the launch status.
  static const bool lds_opt_in = [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&tq_flat_kernel<QG, BS, TQ4>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    (void)hipGetLastError();
    return true;
  }();
  (void)lds_opt_in;
  hipLaunchKernelGGL((tq_flat_kernel<QG, BS, TQ4>), dim3((unsigned)a.n_groups),
                     dim3(64 * kFlatWaves), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_flat(const FlatArgs& a, int query_group_size, int kv_block_size, bool tq4,
                       hipStream_t stream) {
  TQ_DISPATCH(launch_flat_t, query_group_size, kv_block_size, tq4, a, stream);
}

template <int QG, int BS, bool TQ4>
hipError_t launch_partition_t(const PartitionArgs& a, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((tq_partition_kernel<QG, BS, TQ4>), grid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

template <int QG, int BS, bool TQ4>
hipError_t launch_partition_flat_t(const PartitionArgs& a, int n_groups, hipStream_t stream) {
  if constexpr (!TQ4) {
    // The plan chooses this kernel for the 4-bit format only; no fp8 instance is built.
    (void)a, (void)n_groups, (void)stream;
    return hipErrorInvalidValue;
  } else {
    constexpr size_t lds = (size_t)kFlatWaves * kWaveLds;
    static_assert(lds + kTq4TableEntries * 4 * tq4_flat_table_cols(TQ4) + 1024 <= 160 * 1024,
                  "LDS per workgroup");
    // Dynamic LDS beyond 64 KiB needs the opt-in, once; an error here only means
    // the runtime needs none, and must not leak into the launch status.
    static const bool lds_opt_in = [] {
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&tq_partition_flat_kernel<QG, BS, TQ4>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      (void)hipGetLastError();
      return true;
    }();
    (void)lds_opt_in;
    hipLaunchKernelGGL((tq_partition_flat_kernel<QG, BS, TQ4>), dim3((unsigned)n_groups),
                       dim3(64 * kFlatWaves), lds, stream, a);
    return hipGetLastError();
  }
}

hipError_t launch_partition(PartitionArgs a, int num_seqs, int query_group_size,
                            int kv_block_size, bool tq4, hipStream_t stream) {
  a.num_seqs = num_seqs;
  a.nt_partials = partials_nontemporal(num_seqs, a.st.num_kv_heads, a.num_partitions,
                                       query_group_size, tq4) ? 1 : 0;
  const int flat_groups = plan_partition_flat_groups(num_seqs, a.st.num_kv_heads, a.len_cap,
                                                     a.partition_tokens, tq4, device_cu_count());
  if (flat_groups > 0) {
    a.parts_per_wave = 0;  // unused by the flat kernel
    TQ_DISPATCH(launch_partition_flat_t, query_group_size, kv_block_size, tq4, a, flat_groups, stream);
  }
  const int64_t units = (int64_t)num_seqs * a.st.num_kv_heads * a.num_partitions;
  a.parts_per_wave = choose_parts_per_wave(units, a.num_partitions);
  const int64_t groups = (a.num_partitions + a.parts_per_wave - 1) / a.parts_per_wave;
  const dim3 grid((unsigned)(num_seqs * (int64_t)a.st.num_kv_heads * groups));
  a.rotate = rotate_units(grid.x, device_cu_count()) ? 1 : 0;
  TQ_DISPATCH(launch_partition_t, query_group_size, kv_block_size, tq4, a, grid, stream);
}

template <int QG, int BS, bool TQ4>
hipError_t launch_fused_t(const FusedArgs& a, unsigned grid, int waves, hipStream_t stream) {
  // Allow dynamic LDS beyond 64 KiB for this kernel, once; an error here only
  // means the runtime needs no opt-in, and must not leak into the launch status.
  static const bool lds_opt_in = [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&tq_fused_kernel<QG, BS, TQ4>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 8 * kWaveLds);
    (void)hipGetLastError();
    return true;
  }();
  (void)lds_opt_in;
  hipLaunchKernelGGL((tq_fused_kernel<QG, BS, TQ4>), dim3(grid), dim3(64 * waves),
                     (size_t)waves * kWaveLds, stream, a);
  return hipGetLastError();
}

hipError_t launch_fused(const FusedArgs& a_in, int num_seqs, int waves, int query_group_size,
                        int kv_block_size, bool tq4, hipStream_t stream) {
  FusedArgs a = a_in;
  const unsigned grid = (unsigned)((int64_t)num_seqs * a.st.num_kv_heads * a.splits);
  a.rotate = rotate_units((int64_t)grid * waves, device_cu_count()) ? 1 : 0;
  TQ_DISPATCH(launch_fused_t, query_group_size, kv_block_size, tq4, a, grid, waves, stream);
}

#undef TQ_DISPATCH

hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.num_tokens * a.num_kv_heads;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(tq_kv_write_kernel, dim3((unsigned)((rows + kKvRowsPerWg - 1) / kKvRowsPerWg)),
                     dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_validate(const ValidateArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(tq_validate_kernel, dim3((unsigned)a.num_seqs), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_reduce(const ReduceArgs& a, int num_seq_heads, hipStream_t stream) {
  hipLaunchKernelGGL(tq_merge_kernel, dim3(num_seq_heads), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tq
