// Absorbed MLA over packed fp8 latents for decode batches (DSA resource page: attend;
// ttnn.transformer.sparse_sdpa operation line, kv parameter for the 656-byte row): for row t and
// head h over the row's picked positions j,
//   logit_j = sm_scale * (q_nope[h] . c_j[0:512] + q_pe[h] . kpe_j),
//   out[h]  = sum_j softmax(logit)_j * c_j[0:512],
// with c_j[d] = e4m3(code_j[d]) * scale_j[d / 128] and kpe_j the row's 64 bf16 rope values.
//
// A decode batch has few rows, so a row's picks are split over workgroups to fill the chip, and
// each split's partial output costs HEADS x 512 values. A workgroup here takes 32 heads (a
// quarter of the partial of a 128-head workgroup) and up to 512 picks, in steps of 4 tiles of 32
// keys, over eight waves: wave (hf, c) = (w / 4, w % 4) takes heads 16 hf .. +15, scores tile c
// of each step (Q.K^T) and forms output columns 128 c .. +127 of its heads over all 4 tiles
// (P.V), both with v_mfma_f32_16x16x32_bf16. Column block c is exactly the keys' fp8 scale group
// c. Sixteen heads a wave keep the query operand at 64 + 8 registers and the accumulators at 32,
// so two waves share a SIMD and hide each other's LDS reads and code widening. Per step the
// waves exchange through LDS the tile maxima per head (one common running max per head, raised
// only past 2^8 of headroom, so all four waves of a head half rescale identically) and P in fp32
// (each reader folds its own group scale in and rounds once to bf16 for the matrix cores).
// Per tile:
//   gather  the tile's codes (16-byte piece p of key row r at slot p ^ (r & 15), two rows per 1 KB
//           DMA) and group scales (fp32, group-major) go from HBM straight into LDS
//           (global_load_lds), each of the tile's two waves issuing half the rows and one of the
//           two scale instructions, one step ahead; the rope values go from HBM straight into the
//           registers of both waves, one tile ahead.
//   Q.K^T   A = keys (16 rows of the tile a block, lane (l16, G): row 16m + l16, pieces 4J + G of
//           its codes: dims 64J + 16G .. +16, two k-steps) widened exactly to bf16 in registers,
//           B = queries in the same dim order. Each 128-dim group accumulates apart and is scaled
//           per key in fp32 (exact); the rope steps are unscaled. D lane (l16, G): head l16, keys
//           16m + 4G + i.
//   P.V     A = P of tile u (lane: head l16, keys 8G .. +8) times the group-c scales; B = codes read
//           transposed (ds_read_b64_tr_b8, lane: column 128c + 16n + l16, keys 8G .. +8) and
//           widened. D lane (l16, G): column 16n + l16, heads 4G + i.
// Picks of -1 (or outside the row's causal range) load the row's own latent and get weight 0.
#include <stddef.h>

#include "dsa_internal.hpp"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int R = 512, PR = 64;
constexpr int kRowBytes = R + 16 + 2 * PR;    // 656: codes, 4 fp32 scales, bf16 rope
constexpr int kScaleOff = R, kRopeOff = R + 16;
constexpr int CH = 32;                        // keys per tile
constexpr int HPB = 32;                       // heads per workgroup
constexpr int kMaxPicks = 512;                // picks per workgroup
constexpr float kLazy = 8.0f;                 // log2 headroom before O is rescaled

constexpr int kCodeBytes = CH * R;            // 16 KB: a tile's codes
constexpr int kSlot = kCodeBytes + 4 * CH * 4;   // + group-major fp32 scales
static_assert(kSlot % 512 == 0, "slots start on 512-byte boundaries");
constexpr int kQtPitch = R * 2 + 16;          // LDS pitch of a staged q_nope row (65 bank groups)
constexpr int kOutPitch = 128 * 2 + 16;       // a head's 128 output columns, bf16

__device__ __forceinline__ void dma16(const void* src, uint32_t m0) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void dma4(const void* src, uint32_t m0) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" : : "v"(src), "{m0}"(m0) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}
// LDS reads of a slot are done before a DMA refills it
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p));
}
__device__ __forceinline__ bf16x8 lds_bf16x8(uint32_t a) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(static_cast<uintptr_t>(a));
}
__device__ __forceinline__ u32x4 lds_u32x4(uint32_t a) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(static_cast<uintptr_t>(a));
}
__device__ __forceinline__ f32x4 lds_f32x4(uint32_t a) {
  return *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(static_cast<uintptr_t>(a));
}
__device__ __forceinline__ i32x2 lds_tr8(uint32_t a) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      reinterpret_cast<i32x2 __attribute__((address_space(3)))*>(static_cast<uintptr_t>(a)));
}

// 8 e4m3 codes (two little-endian words) -> bf16, exactly
__device__ __forceinline__ bf16x8 widen_e4m3(uint32_t w0, uint32_t w1) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  const bf16x4 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  const bf16x4 cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kCols = 4;                       // tiles per step = output column blocks
constexpr int kHH = 16;                        // heads per wave
constexpr int kPPitch = CH * 4 + 16;           // LDS pitch of a head's P (fp32, 32 keys)

struct Smem {
  uint8_t ring[kCols][2][kSlot];               // tile c's two slots
  uint8_t pbuf[2][kCols][kHH * kPPitch];       // P of tile c for head half hf
  int tok[2][kMaxPicks];                       // per head half: pool token of each pick (~own if not real)
  float mx[kCols][2][kHH];
  float lsum[kCols][2][kHH];
  int last[kWaves];
};
static_assert(sizeof(Smem) <= 160 * 1024, "LDS budget");
static_assert(kWaves * kHH * kOutPitch <= int(sizeof(Smem::ring)), "output staging fits in the ring");
static_assert(8 * kQtPitch <= kSlot, "eight staged query rows fit in a slot");

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// the largest of x over lanes l, l ^ 16, l ^ 32, l ^ 48 (sum when ADD)
template <bool ADD>
__device__ __forceinline__ float quad_reduce(float x) {
  const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = ADD ? __uint_as_float(s32[0]) + __uint_as_float(s32[1])
          : fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
  const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return ADD ? __uint_as_float(s16[0]) + __uint_as_float(s16[1])
             : fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
}

__global__ void __launch_bounds__(kThreads, 1)
attend_f8_split(DevPlan p, const int32_t* __restrict__ sel, const uint8_t* __restrict__ q_nope,
                const uint8_t* __restrict__ q_pe, const uint8_t* __restrict__ pool, float scale_log2,
                const float* __restrict__ sink, uint16_t* __restrict__ out,
                uint16_t* __restrict__ part_o, float* __restrict__ part_ml, int topk, int H,
                int n_splits, int per, int log2_ps) {
  __shared__ __attribute__((aligned(1024))) Smem sm;
  const int t = blockIdx.x;
  const int h0 = blockIdx.y * HPB;
  const int split = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hf = wave >> 2, c = wave & 3;
  const int l16 = lane & 15, G = lane >> 4;
  const int l32 = lane & 31, g = lane >> 5;
  const uint32_t sm0 = lds_u32(&sm);

  // ---- set-up. The picks of the wave's tiles c, c + 4, ... (the same in both head halves: each
  // half keeps its own copy of their tokens) and the span head the longest chain (picks and span
  // -> page table -> gather) and go first, then the sink and the queries (four 1 KB q_nope rows a
  // wave, staged; q_pe straight into the B operand of the rope steps: lane (l16, G), head
  // 16 hf + l16, dims 32j + 8G .. +8), whose 8 MB over the chip the span lookup need not wait for.
  const int k0 = split * per;
  const int npk = max(0, min(topk, k0 + per) - k0);
  int jv[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int i = (c + kCols * (g + 2 * r)) * CH + l32;
    jv[r] = i < npk ? sel[int64_t(t) * topk + k0 + i] : -1;
  }
  const dsa_span span0 = dsa::span_chunk(p.spans, p.n_spans, 0);
  const float sink_raw = sink != nullptr ? sink[h0 + kHH * hf + l16] : -__builtin_inff();
  asm volatile("" ::: "memory");   // the queries' loads stay behind these
  u32x4 qt[HPB / kWaves];
  {
    const uint8_t* qn = q_nope + (int64_t(t) * H + h0 + (HPB / kWaves) * wave) * R * 2 + 16 * lane;
#pragma unroll
    for (int i = 0; i < HPB / kWaves; ++i) qt[i] = *reinterpret_cast<const u32x4*>(qn + i * R * 2);
  }
  bf16x8 qpe[2];
  {
    const uint8_t* qp = q_pe + ((int64_t(t) * H + h0 + kHH * hf + l16) * PR + 8 * G) * 2;
#pragma unroll
    for (int j = 0; j < 2; ++j) qpe[j] = *reinterpret_cast<const bf16x8*>(qp + 64 * j);
  }
  dsa_span sp;
  dsa::row_span_from(span0, p.spans, p.n_spans, t, &sp);
  const float sk_in = sink_raw == -__builtin_inff() ? sink_raw : sink_raw * scale_log2;
  const int pos = sp.ctx_start + (t - sp.q_start);
  int own, ptok[2];
  {
    int off;
    const int pg = dsa::page_of(p, sp, pos, &off);
    own = (pg << log2_ps) + off;
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int j = jv[r] >= 0 && jv[r] <= pos ? jv[r] : pos;
    int off;
    const int pg = dsa::page_of(p, sp, j, &off);
    ptok[r] = (pg << log2_ps) + off;
  }
  asm volatile("" :: "v"(ptok[0]), "v"(ptok[1]), "v"(own));   // one wait for all of them
  const int npk_tiles = (npk + CH - 1) / CH * CH;
  int last = -1;
  uint32_t vb[4];   // real-pick bits of tiles c + 4k, k = 0 .. 3 (bit r: row r)
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int i = (c + kCols * (g + 2 * r)) * CH + l32;
    const bool real = jv[r] >= 0 && jv[r] <= pos;
    if (real) last = i;
    if (i < npk_tiles) sm.tok[hf][i] = real ? ptok[r] : ~own;
    const uint64_t bits = __builtin_amdgcn_ballot_w64(real);
    vb[2 * r] = uint32_t(bits);
    vb[2 * r + 1] = uint32_t(bits >> 32);
  }
  for (int o = 32; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o));
  if (lane == 0) sm.last[wave] = last;
  auto in_range = [&](int k) { return (c + kCols * k) * CH < npk_tiles; };

  const uint32_t ring0 = sm0 + uint32_t(offsetof(Smem, ring));
  auto slot_of = [&](int cc, int b) { return ring0 + uint32_t((2 * cc + b) * kSlot); };
  const int* tokp = sm.tok[hf];
  auto tok_at = [&](int idx) {
    const int v = tokp[idx];
    return v < 0 ? ~v : v;
  };
  // this wave's half of the gather of tile (c, k) into slot b: rows 16 hf .. +15, two a 1 KB
  // instruction (16-byte piece p of row r at p ^ (r & 15)), and group-scale instruction hf
  // (lane l: group 2 hf + l / 32 of row l % 32; the scales are group-major)
  auto issue_codes = [&](int k, int b) {
    const int c0 = (c + kCols * k) * CH;
    const uint32_t dst = slot_of(c, b);
    int tk[CH / 4];
#pragma unroll
    for (int i = 0; i < CH / 4; ++i) tk[i] = tok_at(c0 + kHH * hf + 2 * i + g);
    const int tks = tok_at(c0 + l32);
    wait_lgkm0();   // the tokens are read, and so is whatever this slot held
#pragma unroll
    for (int i = 0; i < CH / 4; ++i) {
      // row 16 hf + 2i + g, piece l32 ^ (2i + g); the offset is recomputed at each use rather
      // than kept as eight 64-bit addresses across the loop
      uint32_t lo = uint32_t(16 * (l32 ^ (2 * i + g)));
      asm volatile("" : "+v"(lo));
      dma16(pool + (int64_t(tk[i]) * kRowBytes + lo), dst + uint32_t(1024 * ((CH / 4) * hf + i)));
    }
    dma4(pool + int64_t(tks) * kRowBytes + kScaleOff + 4 * (2 * hf + g), dst + uint32_t(kCodeBytes + 256 * hf));
  };
  // rope values of tile (c, k) as the A operand of the rope steps: block m, lane (l16, G) holds
  // row 16m + l16, dims 32j + 8G .. +8 in rp[m][j]
  auto load_rope = [&](int k, bf16x8 (&rp)[2][2]) {
    const int c0 = (c + kCols * k) * CH;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint8_t* src = pool + int64_t(tok_at(c0 + 16 * m + l16)) * kRowBytes + kRopeOff + 16 * G;
#pragma unroll
      for (int j = 0; j < 2; ++j) rp[m][j] = *reinterpret_cast<const bf16x8*>(src + 64 * j);
    }
  };
  // The first tile's gather into slot 0 (whenever the tile is in range, so that a slot a step
  // reads holds finite values) and its rope values go out first, then the q_nope rows (in by now:
  // they were requested with the picks) are staged, head h in slot (h / 8, 1). The barriers from
  // here on order LDS traffic only: each wave waits for its own gathers (their vector-memory
  // count) before the barrier after which the other wave of the tile reads them.
  bf16x8 rp[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int j = 0; j < 2; ++j) rp[m][j] = bf16x8{};
  if (in_range(0)) {
    issue_codes(0, 0);
    load_rope(0, rp);
  }
  auto stage_row = [&](int h) { return slot_of(h / 8, 1) + uint32_t((h % 8) * kQtPitch); };
#pragma unroll
  for (int i = 0; i < HPB / kWaves; ++i)
    *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(
        uintptr_t(stage_row((HPB / kWaves) * wave + i) + 16 * lane)) = qt[i];
  dsa::lds_barrier();
  // the B operand of the queries: lane (l16, G), k-steps 2J and 2J + 1 = dims 64J + 16G .. +8 and
  // + 8 .. +16 of head 16 hf + l16
  bf16x8 qb[R / 32];
  {
    const uint32_t row = stage_row(kHH * hf + l16) + uint32_t(32 * G);
#pragma unroll
    for (int J = 0; J < R / 64; ++J) {
      qb[2 * J] = lds_bf16x8(row + 128 * J);
      qb[2 * J + 1] = lds_bf16x8(row + 128 * J + 16);
    }
  }
  int n_tiles = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) n_tiles = max(n_tiles, (sm.last[w] + CH) / CH);
  n_tiles = __builtin_amdgcn_readfirstlane(n_tiles);
  const int n_steps = (n_tiles + kCols - 1) / kCols;
  // tile c of step k is workgroup tile c + 4k, present while below n_tiles
  auto has = [&](int cc, int k) { return cc + kCols * k < n_tiles; };
  dsa::lds_barrier();   // every wave has its query operand: the slots 1 may be overwritten

  f32x4 o[8];   // O[head 4G + i][column 128c + 16n + l16] in o[n][i]
#pragma unroll
  for (int n = 0; n < 8; ++n) o[n] = f32x4{};
  float m_run = -__builtin_inff();   // common running max of head l16 (log2 units)
  float l_run = 0.0f;                // this lane's part of the sum over the wave's keys

  // Per-lane LDS offsets. Q.K^T A: row r = 16m + l16 (r & 15 = l16), piece 4J + G at
  // 16 ((4J + G) ^ l16) = a_lane ^ 64J. P.V B: row 8G + l16 / 2, half l16 % 2 of piece 8c + n at
  // 16 ((8c + n) ^ (r & 15)) = tr_lane ^ 16n.
  const uint32_t a_lane = uint32_t((l16 >> 1) * 1024 + (l16 & 1) * 512 + 64 * (l16 >> 2) + 16 * (G ^ (l16 & 3)));
  const int tr_row = 8 * G + (l16 >> 1);
  const int trx = tr_row & 15;
  const uint32_t tr_lane = uint32_t((tr_row >> 1) * 1024 + (tr_row & 1) * 512 +
                                    16 * (((8 * c) ^ (trx & 8)) | (trx & 7)) + 8 * (l16 & 1));
  const uint32_t pbuf0 = sm0 + uint32_t(offsetof(Smem, pbuf)) + uint32_t(hf * kCols * kHH * kPPitch + l16 * kPPitch);

#pragma clang loop unroll(disable)
  for (int k = 0; k < n_steps; ++k) {
    const int b = k & 1;
    const bool mine = has(c, k);
    // everything this wave has in flight is tile k's (its gather and rope values): an
    // unconditional wait, so that no later use of the rope registers waits again (the gathers
    // are not counted by the compiler, and a wait for the rope values issued after the next
    // tile's gather would hold that gather too)
    wait_vmcnt<0>();
    dsa::lds_barrier();   // the step's tiles are in; every wave is done with step k - 1
    // tile c of step k + 1 into the slot of step k - 1 (at step 0: the staged queries' slot)
    if (has(c, k + 1)) issue_codes(k + 1, b ^ 1);
    f32x4 x[2];
    if (mine) {
      const uint32_t cb = slot_of(c, b);
      // ---- Q.K^T: 32 keys x 16 heads; the rope steps (unscaled) first
      x[0] = f32x4{};
      x[1] = f32x4{};
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int m = 0; m < 2; ++m) x[m] = mfma16(rp[m][j], qpe[j], x[m]);
      // group gg = pairs 2gg, 2gg + 1, accumulated apart and scaled per key in fp32; the pieces
      // and scales of group gg + 1 are requested before group gg's products
      const uint32_t ca = cb + a_lane;
      auto read_group = [&](int gg, u32x4 (&rw)[2][2], f32x4 (&sc)[2]) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int m = 0; m < 2; ++m) rw[jj][m] = lds_u32x4((ca + uint32_t(8192 * m)) ^ uint32_t(64 * (2 * gg + jj)));
#pragma unroll
        for (int m = 0; m < 2; ++m) sc[m] = lds_f32x4(cb + uint32_t(kCodeBytes + 128 * gg + 64 * m + 16 * G));
      };
      u32x4 rw[2][2][2];
      f32x4 sc[2][2];
      read_group(0, rw[0], sc[0]);
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        if (gg + 1 < 4) read_group(gg + 1, rw[(gg + 1) & 1], sc[(gg + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
        f32x4 acc[2] = {f32x4{}, f32x4{}};
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int J = 2 * gg + jj;
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            const u32x4 raw = rw[gg & 1][jj][m];
            acc[m] = mfma16(widen_e4m3(raw[0], raw[1]), qb[2 * J], acc[m]);
            acc[m] = mfma16(widen_e4m3(raw[2], raw[3]), qb[2 * J + 1], acc[m]);
          }
        }
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[m][i] = fmaf(sc[gg & 1][m][i], acc[m][i], x[m][i]);
        __builtin_amdgcn_sched_barrier(0);
      }
      // the next tile's rope values (the rope registers were free since the rope steps)
      if (has(c, k + 1)) load_rope(k + 1, rp);
      // keys that are not real picks score -inf
      const uint32_t tv = k == 0 ? vb[0] : k == 1 ? vb[1] : k == 2 ? vb[2] : vb[3];
      if (tv != 0xFFFFFFFFu) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (!((tv >> (16 * m + 4 * G + i)) & 1u)) x[m][i] = -__builtin_inff();
      }
      float mx = x[0][0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i >> 2][i & 3]);
      mx = quad_reduce<false>(mx);
      if (lane < kHH) sm.mx[c][hf][lane] = mx;
    } else if (lane < kHH) {
      sm.mx[c][hf][lane] = -__builtin_inff();
    }
    dsa::lds_barrier();   // tile maxima in

    // ---- common running max of the head half (the same in its four waves), rescale, P
    float tmax = sm.mx[0][hf][l16];
#pragma unroll
    for (int cc = 1; cc < kCols; ++cc) tmax = fmaxf(tmax, sm.mx[cc][hf][l16]);
    const float mc = tmax * scale_log2;
    float alpha = 1.0f;
    if (mc > m_run + kLazy) {
      alpha = m_run != -__builtin_inff() ? __builtin_amdgcn_exp2f(m_run - mc) : 1.0f;
      m_run = mc;
      l_run *= alpha;
    }
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float av = __shfl(alpha, 4 * G + i);
#pragma unroll
        for (int n = 0; n < 8; ++n) o[n][i] *= av;
      }
    }
    if (mine) {
      const float mneg = m_run != -__builtin_inff() ? -m_run : 0.0f;
      f32x4 pv[2];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pv[m][i] = __builtin_amdgcn_exp2f(fmaf(x[m][i], scale_log2, mneg));
          l_run += pv[m][i];
        }
      const uint32_t pw = pbuf0 + uint32_t(c * kHH * kPPitch + 16 * G);
      *reinterpret_cast<__attribute__((address_space(3))) f32x4*>(uintptr_t(pw)) = pv[0];
      *reinterpret_cast<__attribute__((address_space(3))) f32x4*>(uintptr_t(pw + 64)) = pv[1];
    }
    dsa::lds_barrier();   // P of every tile in

    // ---- P.V over the step's tiles, without branches: a tile past the last reads the step's
    // first tile (always present) with P = 0. Every tile's P (times the group-c scales) first, then
    // the transposed reads of tile u + 1 go out before tile u's products.
    bf16x8 pa[kCols];
#pragma unroll
    for (int u = 0; u < kCols; ++u) {
      const bool pres = has(u, k);
      const int uu = pres ? u : 0;
      const uint32_t pr = pbuf0 + uint32_t(uu * kHH * kPPitch + 32 * G);
      const uint32_t su = slot_of(uu, b) + uint32_t(kCodeBytes + 128 * c + 32 * G);
      const f32x4 p0 = lds_f32x4(pr), p1 = lds_f32x4(pr + 16);
      const f32x4 s0 = lds_f32x4(su), s1 = lds_f32x4(su + 16);
      const float z = pres ? 1.0f : 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pa[u][i] = (__bf16)(p0[i] * s0[i] * z);
        pa[u][4 + i] = (__bf16)(p1[i] * s1[i] * z);
      }
    }
    auto read_tr = [&](int u, i32x2 (&v)[8]) {
      const uint32_t trb = slot_of(has(u, k) ? u : 0, b) + tr_lane;
#pragma unroll
      for (int n = 0; n < 8; ++n) v[n] = lds_tr8(trb ^ uint32_t(16 * n));
    };
    i32x2 tv8[2][8];
    read_tr(0, tv8[0]);
#pragma unroll
    for (int u = 0; u < kCols; ++u) {
      if (u + 1 < kCols) read_tr(u + 1, tv8[(u + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int n = 0; n < 8; ++n)
        o[n] = mfma16(pa[u], widen_e4m3(uint32_t(tv8[u & 1][n][0]), uint32_t(tv8[u & 1][n][1])), o[n]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  wait_vmcnt<0>();

  // ---- output: the head's sum over the half's four waves, then columns 128c .. +127 of the
  // wave's 16 heads, normalised per head (a split's partial by its own sum; the row's output by
  // sum + sink), as bf16 through LDS into 256-byte row pieces
  const float lw = quad_reduce<true>(l_run);
  if (lane < kHH) sm.lsum[c][hf][lane] = lw;
  dsa::lds_barrier();   // also: every wave is done with the ring (its gathers waited for above)
  float L = 0.0f;
#pragma unroll
  for (int cc = 0; cc < kCols; ++cc) L += sm.lsum[cc][hf][l16];
  const float M = m_run;
  float inv_h;
  if (n_splits > 1 || sk_in == -__builtin_inff()) {
    inv_h = L > 0.0f ? 1.0f / L : 0.0f;
  } else if (M == -__builtin_inff()) {
    inv_h = 0.0f;
  } else {
    const float Mx = fmaxf(M, sk_in);
    const float a = __builtin_amdgcn_exp2f(M - Mx);
    inv_h = a / fmaf(L, a, __builtin_amdgcn_exp2f(sk_in - Mx));
  }
  uint8_t* ob = &sm.ring[0][0][0] + wave * kHH * kOutPitch;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hr = 4 * G + i;
    const float inv = __shfl(inv_h, hr);
#pragma unroll
    for (int n = 0; n < 8; ++n)
      reinterpret_cast<uint16_t*>(ob + hr * kOutPitch)[16 * n + l16] = dsa::f32_to_bf16(o[n][i] * inv);
  }
  wait_lgkm0();   // this wave's staging is written (each wave reads back only its own)
  uint16_t* dst = n_splits == 1 ? out + (int64_t(t) * H + h0 + kHH * hf) * R
                                : part_o + ((int64_t(t) * n_splits + split) * H + h0 + kHH * hf) * R;
  // instruction i: heads 4i .. 4i + 3 of the wave, lane = 16-byte piece l16 of head 4i + G
#pragma unroll
  for (int i = 0; i < kHH / 4; ++i) {
    const int hl = 4 * i + G;
    const u32x4 val = *reinterpret_cast<const u32x4*>(ob + hl * kOutPitch + 16 * l16);
    *reinterpret_cast<u32x4*>(dst + int64_t(hl) * R + 128 * c + 8 * l16) = val;
  }
  if (n_splits > 1 && c == 0 && lane < kHH) {
    const int64_t prow = (int64_t(t) * n_splits + split) * H + h0 + kHH * hf + lane;
    part_ml[2 * prow] = M;
    part_ml[2 * prow + 1] = L;
  }
}

}  // namespace

// Split count for the decode kernel: picks per workgroup at most kMaxPicks, then halved until the
// grid (rows x head groups x splits) covers the chip's 256 CUs, keeping at least 128 picks each.
int attend_split_count(const PlanInfo& in, int H, int topk) {
  int s = 1;
  while ((topk + s - 1) / s > kMaxPicks) s *= 2;
  const int base = in.n_rows * (H / HPB);
  while (base * s < 256 && (topk + 2 * s - 1) / (2 * s) >= 128 && s < 16) s *= 2;
  return s;
}

bool attend_split_supported(const dsa_config& c) {
  return c.latent_fmt == DSA_FMT_FP8 && c.q_fmt == DSA_FMT_BF16 && c.kv_lora_rank == R &&
         c.rope_dim == PR && c.n_heads % HPB == 0;
}

hipError_t launch_attend_combine(int S, bool q8, const uint16_t* part_o, const float* part_ml,
                                 const float* sink, float scale_log2, void* out, int n_rows, int H,
                                 hipStream_t st);

hipError_t launch_attend_split(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                               const int32_t* sel, const void* qn, const void* qp, const void* pool,
                               float sm_scale, const float* sink, void* out, void* ws, int log2_ps,
                               hipStream_t st) {
  const dsa_config& c = h->cfg;
  const int s = attend_split_count(in, c.n_heads, c.topk);
  const int per = (c.topk + s - 1) / s;
  uint16_t* part_o = nullptr;
  float* part_ml = nullptr;
  if (s > 1) {
    const size_t rows = size_t(in.n_rows) * s * c.n_heads;
    part_o = static_cast<uint16_t*>(ws);
    part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + ((rows * R * 2 + 255) & ~size_t(255)));
  }
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  dim3 grid(in.n_rows, c.n_heads / HPB, s);
  hipLaunchKernelGGL(attend_f8_split, grid, dim3(kThreads), 0, st, p, sel,
                     static_cast<const uint8_t*>(qn), static_cast<const uint8_t*>(qp),
                     static_cast<const uint8_t*>(pool), scale_log2, sink,
                     static_cast<uint16_t*>(out), part_o, part_ml, c.topk, c.n_heads, s, per, log2_ps);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || s == 1) return e;
  return launch_attend_combine(s, false, part_o, part_ml, sink, scale_log2, out, in.n_rows, c.n_heads, st);
}
