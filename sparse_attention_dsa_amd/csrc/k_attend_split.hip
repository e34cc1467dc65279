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
// keys: in a step, wave w scores its own tile (Q.K^T for the 32 heads) and every wave then forms
// its own 128 output columns (P.V) over all 4 tiles. Column block w is exactly the keys' fp8 scale
// group w, and a wave's output accumulators are 32 x 128 (64 registers), so nothing has to be
// merged at the end. Per step the waves exchange through LDS:
//   the tile maxima per head (one common running max, raised only past 2^8 of headroom, so the
//   four waves rescale identically), and P in fp32, in two halves of 16 keys (each reader folds
//   its own group scale in and rounds once to bf16 for the matrix cores).
// Per tile:
//   gather  the tile's codes (16-byte piece p of key row r at slot p ^ (r & 15), two rows per 1 KB
//           DMA), group scales (fp32, group-major) and rope values (piece p at p ^ (r & 7)) go from
//           HBM straight into LDS (global_load_lds); a wave has two tiles in flight.
//   Q.K^T   v_mfma_f32_32x32x16_bf16, A = the keys as raw codes (16 per lane: two k-steps) widened
//           exactly to bf16 in registers, B = the queries (VGPRs); lane half g of a k-step pair
//           takes dims 32j + 16g .. +16. Each 128-dim group accumulates apart and is scaled per
//           key in fp32 (exact); the rope steps are unscaled.
//   P.V     v_mfma_f32_32x32x16_bf16, A = P (a lane holds one head and 8 keys per k-step), B = the
//           keys' codes read transposed (ds_read_b64_tr_b8: 8 keys of one column per lane) and
//           widened. For the 8 keys of a lane's k-step to be 8 consecutive LDS rows, Q.K^T row m
//           reads LDS row rho(m), m with bits 2 and 3 swapped.
// Picks of -1 (or outside the row's causal range) load the row's own latent and get weight 0.
#include <stddef.h>

#include "dsa_internal.hpp"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int R = 512, PR = 64;
constexpr int kRowBytes = R + 16 + 2 * PR;    // 656: codes, 4 fp32 scales, bf16 rope
constexpr int kScaleOff = R, kRopeOff = R + 16;
constexpr int CH = 32;                        // keys per tile
constexpr int HPB = 32;                       // heads per workgroup
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxPicks = 512;                // picks per workgroup
constexpr float kLazy = 8.0f;                 // log2 headroom before O is rescaled

constexpr int kCodeBytes = CH * R;            // 16 KB: a tile's codes
constexpr int kSlot = kCodeBytes + 4 * CH * 4;   // + group-major fp32 scales
static_assert(kSlot % 512 == 0, "slots start on 512-byte boundaries");
constexpr int kRope = CH * PR * 2;            // 4 KB: a tile's rope values
constexpr int kQtPitch = R * 2 + 16;          // LDS pitch of a staged q_nope row (65 bank groups)
constexpr int kDmaCodes = CH / 2 + 2;         // code and scale instructions per tile
constexpr int kDmaRope = CH * PR * 2 / 1024;  // rope instructions per tile

struct Smem {
  uint8_t ring[kWaves][2][kSlot];             // wave w's two tile slots
  uint8_t rope[kWaves][kRope];                // wave w's rope slot (one tile)
  f32x4 pbuf[kWaves][2][64];                  // P of wave w's tile, one half (16 keys) at a time
  int tok[kMaxPicks];                         // pool token of each pick (~own token if not real)
  uint32_t valid[kMaxPicks / CH];             // per tile: bit r set if row r is a real pick
  float mx[kWaves][HPB];                      // this step's tile maxima per head
  float lsum[kWaves][HPB];                    // each wave's share of the softmax sums
  int last[kWaves];
};
static_assert(sizeof(Smem) <= 160 * 1024, "LDS budget");
// the query staging (first) and the output staging (last) reuse the ring
constexpr int kOutPitch = 128 * 2 + 16;       // a head's 128 output columns, bf16
static_assert(kWaves * HPB * kOutPitch <= int(sizeof(Smem::ring)), "output staging fits in the ring");
static_assert(HPB * kQtPitch <= int(sizeof(Smem::ring)), "query staging fits in the ring");

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

// x *= s for a value held in an AGPR, through one temporary VGPR
__device__ __forceinline__ void scale_agpr(float& x, float s) {
  float tmp;
  asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
               : "+a"(x), "=&v"(tmp) : "v"(s));
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

// LDS row that Q.K^T row m reads: m with bits 2 and 3 swapped
__device__ __forceinline__ int rho(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

__global__ void __launch_bounds__(kThreads, 1)
attend_f8_split(DevPlan p, const int32_t* __restrict__ sel, const uint8_t* __restrict__ q_nope,
                const uint8_t* __restrict__ q_pe, const uint8_t* __restrict__ pool, float scale_log2,
                const float* __restrict__ sink, uint16_t* __restrict__ out,
                uint16_t* __restrict__ part_o, float* __restrict__ part_ml, int topk, int H,
                int n_splits, int per, int log2_ps) {
  // 1 KB alignment: every slot (a multiple of 512 bytes) starts on a 512-byte boundary, so the
  // swizzled piece addresses below are a per-lane base XORed with a constant
  __shared__ __attribute__((aligned(1024))) Smem sm;
  const int t = blockIdx.x;
  const int h0 = blockIdx.y * HPB;
  const int split = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const uint32_t sm0 = lds_u32(&sm);

  // ---- set-up. Wave w handles workgroup tiles w, w + 4, ... (its tile of each step). The picks
  // of its tiles head the longest chain (picks, page table, gathers) and go first, then the
  // queries (whole 1 KB rows of q_nope, one per instruction, and q_pe straight into the B operand
  // of the rope steps: lane (l32, g), dims 16u + 8g .. +8) and the sink, then the span; all of
  // them arrive in one round trip. Each wave then looks up the pages of its picks (one round trip
  // for all of them) and starts gathering its first tile at once.
  const int k0 = split * per;
  const int npk = max(0, min(topk, k0 + per) - k0);
  constexpr int kTilesPerWave = kMaxPicks / CH / kWaves;      // 4
  constexpr int kPickPer = kTilesPerWave / 2;                 // picks per lane: tiles g, g + 2, ...
  int jv[kPickPer];
#pragma unroll
  for (int r = 0; r < kPickPer; ++r) {
    const int i = (wave + kWaves * (g + 2 * r)) * CH + l32;
    jv[r] = i < npk ? sel[int64_t(t) * topk + k0 + i] : -1;
  }
  u32x4 qt[HPB / kWaves];
  {
    const uint8_t* qn = q_nope + (int64_t(t) * H + h0 + (HPB / kWaves) * wave) * R * 2 + 16 * lane;
#pragma unroll
    for (int i = 0; i < HPB / kWaves; ++i) qt[i] = *reinterpret_cast<const u32x4*>(qn + i * R * 2);
  }
  bf16x8 qpe[PR / 16];
  {
    const uint8_t* qp = q_pe + (int64_t(t) * H + h0 + l32) * PR * 2 + 16 * g;
#pragma unroll
    for (int u = 0; u < PR / 16; ++u) qpe[u] = *reinterpret_cast<const bf16x8*>(qp + 32 * u);
  }
  const float sink_raw = sink != nullptr ? sink[h0 + l32] : -__builtin_inff();
  dsa_span sp;
  dsa::row_span(p.spans, p.n_spans, t, &sp);
  const float sk_in = sink_raw == -__builtin_inff() ? sink_raw : sink_raw * scale_log2;
  const int pos = sp.ctx_start + (t - sp.q_start);
  // picks as pool tokens; one that is -1 or past the row is stored as ~own (loads the row's own
  // latent, weight 0). Tiles after the workgroup's last real pick are not processed. Every page
  // table read (the row's own and one per pick, a non-pick looking up the row's own position) is
  // unconditional, so that all of them are in flight together.
  int own, ptok[kPickPer];
  {
    int off;
    const int pg = dsa::page_of(p, sp, pos, &off);
    own = (pg << log2_ps) + off;
  }
#pragma unroll
  for (int r = 0; r < kPickPer; ++r) {
    const int j = jv[r] >= 0 && jv[r] <= pos ? jv[r] : pos;
    int off;
    const int pg = dsa::page_of(p, sp, j, &off);
    ptok[r] = (pg << log2_ps) + off;
  }
  asm volatile("" :: "v"(ptok[0]), "v"(ptok[1]), "v"(own));   // one wait for all of them
  const int npk_tiles = (npk + CH - 1) / CH * CH;
  int last = -1;
#pragma unroll
  for (int r = 0; r < kPickPer; ++r) {
    const int i = (wave + kWaves * (g + 2 * r)) * CH + l32;
    const bool real = jv[r] >= 0 && jv[r] <= pos;
    if (real && i < npk_tiles) last = i;
    if (i < npk_tiles) sm.tok[i] = real ? ptok[r] : ~own;
  }
  for (int o = 32; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o));
  // valid bits of this wave's tiles in the split's range (every one of them has tokens)
  if (lane == 0) sm.last[wave] = last;
  auto in_range = [&](int k) { return (wave + kWaves * k) * CH < npk_tiles; };
  for (int k = 0; in_range(k); ++k) {
    const int c = wave + kWaves * k;
    const uint64_t bits = __builtin_amdgcn_ballot_w64(lane < CH && sm.tok[c * CH + lane] >= 0);
    if (lane == 0) sm.valid[c] = uint32_t(bits);
  }

  // ---- gathers of this wave's tile of step k into slot b
  const uint32_t ring0 = sm0 + uint32_t(offsetof(Smem, ring));
  auto slot_of = [&](int w, int b) { return ring0 + uint32_t((2 * w + b) * kSlot); };
  const uint32_t rope_b = sm0 + uint32_t(offsetof(Smem, rope)) + uint32_t(wave * kRope);
  auto tok_at = [&](int idx) {
    const int v = sm.tok[idx];
    return v < 0 ? ~v : v;
  };
  auto issue_codes = [&](int k, int b) {
    const int c0 = (wave + kWaves * k) * CH;
    const uint32_t dst = slot_of(wave, b);
    int tk[CH / 2];
#pragma unroll
    for (int i = 0; i < CH / 2; ++i) tk[i] = tok_at(c0 + 2 * i + (lane >> 5));
    const int tks = tok_at(c0 + l32);
    wait_lgkm0();   // the tokens are read, and so is whatever this slot held
#pragma unroll
    for (int i = 0; i < CH / 2; ++i) {
      const int r = 2 * i + (lane >> 5);
      dma16(pool + int64_t(tk[i]) * kRowBytes + 16 * ((lane & 31) ^ (r & 15)), dst + uint32_t(1024 * i));
    }
    // group scales, group-major: lane l of instruction i takes group 2i + l / 32 of row l % 32
#pragma unroll
    for (int i = 0; i < 2; ++i)
      dma4(pool + int64_t(tks) * kRowBytes + kScaleOff + 4 * (2 * i + (lane >> 5)),
           dst + uint32_t(kCodeBytes + 256 * i));
  };
  auto issue_rope = [&](int k) {
    const int c0 = (wave + kWaves * k) * CH;
    int tk[kDmaRope];
#pragma unroll
    for (int i = 0; i < kDmaRope; ++i) tk[i] = tok_at(c0 + 8 * i + (lane >> 3));
    wait_lgkm0();
#pragma unroll
    for (int i = 0; i < kDmaRope; ++i) {
      const int r = 8 * i + (lane >> 3);
      dma16(pool + int64_t(tk[i]) * kRowBytes + kRopeOff + 16 * ((lane & 7) ^ (r & 7)), rope_b + uint32_t(1024 * i));
    }
  };
  // q_nope rows (in by now: they were requested with the picks): head h in slot 1 of wave h / 8.
  // Each wave then takes the B operand of its k-step pairs: lane (l32, g), pair j = dims 32j + 16g
  // .. +16 of head l32.
  static_assert((HPB / kWaves) * kQtPitch <= kSlot, "a wave's query rows fit in a slot");
  auto stage_row = [&](int h) { return slot_of(h / (HPB / kWaves), 1) + uint32_t((h % (HPB / kWaves)) * kQtPitch); };
#pragma unroll
  for (int i = 0; i < HPB / kWaves; ++i)
    *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(
        uintptr_t(stage_row((HPB / kWaves) * wave + i) + 16 * lane)) = qt[i];
  // the first tile's gather, into slot 0. It goes out whenever the wave's first tile is in range,
  // so that slot 0 holds finite values wherever a step reads it. The barriers from here on order
  // LDS traffic only: a gather is waited for (its vector-memory count) by the wave that issued it,
  // before the barrier after which other waves read it, so no barrier waits for a gather in flight.
  if (in_range(0)) {
    issue_codes(0, 0);
    issue_rope(0);
  }
  dsa::lds_barrier();
  bf16x8 qb[R / 16];
  {
    const uint32_t row = stage_row(l32) + uint32_t(32 * g);
#pragma unroll
    for (int j = 0; j < R / 32; ++j) {
      qb[2 * j] = lds_bf16x8(row + 64 * j);
      qb[2 * j + 1] = lds_bf16x8(row + 64 * j + 16);
    }
  }
  int n_tiles = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) n_tiles = max(n_tiles, (sm.last[w] + CH) / CH);
  n_tiles = __builtin_amdgcn_readfirstlane(n_tiles);
  const int n_steps = (n_tiles + kWaves - 1) / kWaves;
  // wave w's tile of step k is workgroup tile w + 4k, present while below n_tiles
  auto has = [&](int w, int k) { return w + kWaves * k < n_tiles; };
  dsa::lds_barrier();   // every wave has its query operand: the slots 1 may be overwritten
  if (has(wave, 1)) issue_codes(1, 1);

  f32x16 o[4];          // O[head 8*(v/4) + 4*g + v%4][column 128*wave + 32*q + l32]
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  float m_run = -__builtin_inff();   // common running max of head l32 (log2 units)
  float l_run = 0.0f;                // this lane's part of the sum over this wave's keys

  // Per-lane operand addresses. Piece p ^ x of a row sits at 16 (p ^ x) = (32 (p / 2)) ^ 16 ((p % 2)
  // ^ x) bytes: a base holding the row, the lane's half and x, XORed with a constant per step.
  const int rq = rho(l32);
  const uint32_t a_lane = uint32_t((rq >> 1) * 1024 + (rq & 1) * 512 + 16 * (g ^ (rq & 15)));
  const uint32_t rope_a = rope_b + uint32_t(rq * PR * 2 + 16 * (g ^ (rq & 7)));
  // P.V B: row 16s + 8g + (lane % 16) / 2 of a tile, half lane % 2 of the 16 columns of piece
  // 2nt + (lane / 16) % 2
  const int tr_row = 8 * g + ((lane & 15) >> 1);
  const uint32_t tr_lane = uint32_t((tr_row >> 1) * 1024 + (tr_row & 1) * 512 +
                                    16 * (((lane >> 4) & 1) ^ (tr_row & 15)) + 8 * (lane & 1));
  const uint32_t pbuf0 = sm0 + uint32_t(offsetof(Smem, pbuf)) + uint32_t(16 * lane);

#pragma clang loop unroll(disable)
  for (int k = 0; k < n_steps; ++k) {
    const int b = k & 1;
    const bool mine = has(wave, k);
    f32x16 x;
    if (mine) {
      if (k == 0 && has(wave, 1)) wait_vmcnt<kDmaCodes>(); else wait_vmcnt<0>();
      const uint32_t cb = slot_of(wave, b);
      const uint32_t sb = cb + uint32_t(kCodeBytes);
      // ---- Q.K^T: 32 keys x 32 heads; lane holds head l32, rows m = 8*(v/4) + 4*g + v%4
      x = f32x16{};
#pragma unroll
      for (int u = 0; u < PR / 16; ++u)
        x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_bf16x8(rope_a ^ uint32_t(32 * u)), qpe[u], x, 0, 0, 0);
      if (has(wave, k + 1)) issue_rope(k + 1);   // the rope slot is read: refill it
      const uint32_t arow = cb + a_lane;
      auto a_raw = [&](int j) { return lds_u32x4(arow ^ uint32_t(32 * j)); };
      u32x4 ra[3];
      ra[0] = a_raw(0);
      ra[1] = a_raw(1);
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        f32x4 sc[4];
#pragma unroll
        for (int vq = 0; vq < 4; ++vq)
          sc[vq] = lds_f32x4(sb + uint32_t(4 * (CH * gg + 16 * (vq >> 1) + 8 * g + 4 * (vq & 1))));
        f32x16 acc = f32x16{};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int j = 4 * gg + jj;
          if (j + 2 < R / 32) ra[(j + 2) % 3] = a_raw(j + 2);
          const u32x4 cur = ra[j % 3];
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(widen_e4m3(cur[0], cur[1]), qb[2 * j], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(widen_e4m3(cur[2], cur[3]), qb[2 * j + 1], acc, 0, 0, 0);
        }
        // rows 4vq + r of the lane are LDS rows 16(vq/2) + 8g + 4(vq%2) + r
#pragma unroll
        for (int vq = 0; vq < 4; ++vq)
#pragma unroll
          for (int r = 0; r < 4; ++r) x[4 * vq + r] = fmaf(sc[vq][r], acc[4 * vq + r], x[4 * vq + r]);
      }
      // keys that are not real picks score -inf
      const uint32_t tv = sm.valid[wave + kWaves * k];
      if (tv != 0xFFFFFFFFu) {
        const uint32_t tg = tv >> (8 * g);
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (!((tg >> (16 * (v >> 3) + 4 * ((v >> 2) & 1) + (v & 3))) & 1u)) x[v] = -__builtin_inff();
      }
      float mx = x[0];
#pragma unroll
      for (int v = 1; v < 16; ++v) mx = fmaxf(mx, x[v]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if (g == 0) sm.mx[wave][l32] = mx;
    } else if (g == 0) {
      sm.mx[wave][l32] = -__builtin_inff();
    }
    dsa::lds_barrier();   // tile maxima in; every wave is done with the tiles of step k - 1
    // tile k + 1 into the slot of tile k - 1
    if (k >= 1 && has(wave, k + 1)) issue_codes(k + 1, b ^ 1);

    // ---- common running max (the same in every wave), rescale, P of this wave's keys
    float tmax = sm.mx[0][l32];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) tmax = fmaxf(tmax, sm.mx[w][l32]);
    const float mc = tmax * scale_log2;
    float alpha = 1.0f;
    if (mc > m_run + kLazy) {
      alpha = m_run != -__builtin_inff() ? __builtin_amdgcn_exp2f(m_run - mc) : 1.0f;
      m_run = mc;
      l_run *= alpha;
    }
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float av = __shfl(alpha, 8 * (v >> 2) + 4 * g + (v & 3));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float e = o[q][v];
          scale_agpr(e, av);
          o[q][v] = e;
        }
      }
    }
    float pv[16];
    if (mine) {
      const float mneg = m_run != -__builtin_inff() ? -m_run : 0.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        pv[v] = __builtin_amdgcn_exp2f(fmaf(x[v], scale_log2, mneg));
        l_run += pv[v];
      }
    }

    // ---- P.V over the step's tiles, k-step s (keys 16s .. 16s + 15 of every tile) at a time:
    // slot i of lane half g is LDS row 16s + 8g + i, pv[8s + i] in its owner wave
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (mine) {
        sm.pbuf[wave][0][lane] = f32x4{pv[8 * s], pv[8 * s + 1], pv[8 * s + 2], pv[8 * s + 3]};
        sm.pbuf[wave][1][lane] = f32x4{pv[8 * s + 4], pv[8 * s + 5], pv[8 * s + 6], pv[8 * s + 7]};
      }
      dsa::lds_barrier();
      // every source's P and scales first (their latencies overlap), then per source the
      // transposed B reads one source ahead of its four products
      bf16x8 pa[kWaves];
#pragma unroll
      for (int u = 0; u < kWaves; ++u) {
        if (!has(u, k)) continue;
        const uint32_t sbw = slot_of(u, b) + uint32_t(kCodeBytes + 4 * (CH * wave + 16 * s + 8 * g));
        const f32x4 p0 = lds_f32x4(pbuf0 + uint32_t(u * 2048));
        const f32x4 p1 = lds_f32x4(pbuf0 + uint32_t(u * 2048 + 1024));
        const f32x4 s0 = lds_f32x4(sbw), s1 = lds_f32x4(sbw + 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pa[u][i] = (__bf16)(p0[i] * s0[i]);
          pa[u][4 + i] = (__bf16)(p1[i] * s1[i]);
        }
      }
      auto tr_src = [&](int u, i32x2* bt) {
        const uint32_t rbase = slot_of(u, b) + tr_lane + uint32_t(8192 * s);
#pragma unroll
        for (int q = 0; q < 4; ++q) bt[q] = lds_tr8(rbase ^ uint32_t(32 * (4 * wave + q)));
      };
      i32x2 bt[2][4];
      tr_src(0, bt[0]);
#pragma unroll
      for (int u = 0; u < kWaves; ++u) {
        if (!has(u, k)) continue;
        if (u + 1 < kWaves && has(u + 1, k)) tr_src(u + 1, bt[(u + 1) & 1]);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          o[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              pa[u], widen_e4m3(uint32_t(bt[u & 1][q][0]), uint32_t(bt[u & 1][q][1])), o[q], 0, 0, 0);
      }
      if (s == 0) dsa::lds_barrier();   // every wave has read the first half before the second
    }
  }
  wait_vmcnt<0>();

  // ---- output: the sum over all waves' keys, then columns 128w .. +127 of the 32 heads,
  // normalised per head (a split's partial by its own sum; the row's output by sum + sink), as
  // bf16 through LDS into 256-byte row pieces
  const float lw = l_run + __shfl_xor(l_run, 32);
  if (g == 0) sm.lsum[wave][l32] = lw;
  dsa::lds_barrier();   // also: every wave is done with the ring (its gathers waited for above)
  float L = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) L += sm.lsum[w][l32];
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
  uint8_t* ob = &sm.ring[0][0][0] + wave * HPB * kOutPitch;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int hr = 8 * (v >> 2) + 4 * g + (v & 3);
    const float inv = __shfl(inv_h, hr);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      reinterpret_cast<uint16_t*>(ob + hr * kOutPitch)[32 * q + l32] = dsa::f32_to_bf16(o[q][v] * inv);
  }
  wait_lgkm0();   // this wave's staging is written (each wave reads back only its own)
  uint16_t* dst = n_splits == 1 ? out + (int64_t(t) * H + h0) * R
                                : part_o + ((int64_t(t) * n_splits + split) * H + h0) * R;
  // instruction i: heads 4i .. 4i + 3, lane = 16-byte piece (lane % 16) of head 4i + lane / 16
#pragma unroll
  for (int i = 0; i < HPB / 4; ++i) {
    const int hl = 4 * i + (lane >> 4);
    const u32x4 val = *reinterpret_cast<const u32x4*>(ob + hl * kOutPitch + 16 * (lane & 15));
    *reinterpret_cast<u32x4*>(dst + int64_t(hl) * R + 128 * wave + 8 * (lane & 15)) = val;
  }
  if (n_splits > 1 && wave == 0 && g == 0) {
    const int64_t prow = (int64_t(t) * n_splits + split) * H + h0 + l32;
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
