// Absorbed MLA over each row's picked latents on the matrix cores (DSA resource page: attend;
// ttnn.transformer.sparse_sdpa operation line): for row t and head h over picked positions j,
//   logit_j = sm_scale * (q_nope[h] . c_j[0:512] + q_pe[h] . c_j[512:576]),
//   out[h]  = sum_j softmax(logit)_j * c_j[0:512].
// Shapes: 512 + 64 latents (bf16 rows, or packed 656-byte fp8 rows), heads a multiple of 128;
// queries and output bf16, or plain e4m3 (widened exactly to bf16 on load; the output rounded to
// e4m3). An attention sink (ttnn.transformer.sparse_sdpa, attention_sink) adds e^{scale * sink[h]}
// to head h's softmax denominator once, where the row's output is normalised.
//
// A workgroup of 4 waves takes one row, 128 heads and one range of its picks (a split); each wave
// owns 32 heads and all 512 output columns, so waves never exchange softmax state, and every
// latent tile in LDS feeds all 128 heads. Picks are processed in tiles of 32 keys:
//   gather  the tile's latent rows go from HBM straight into LDS (global_load_lds, 16 bytes per
//           lane), a ring of NB tiles deep, so that NB - 1 tiles are in flight while one is used.
//           Rows are stored as a 1024-byte latent part at a pitch of 1072 bytes (67 16-byte bank
//           groups: 16 keys of one Q.K^T read and 4 keys of one transposed read all fall in
//           distinct banks) and a 128-byte rope part per key with its 16-byte pieces XOR-swizzled.
//           fp8 rows land as codes and are converted exactly to bf16 once per tile; their
//           128-element group scales are kept apart.
//   Q.K^T   v_mfma_f32_32x32x16_bf16, A = the 32 keys (LDS), B = the wave's 32 queries (VGPRs,
//           36 steps of 16 dims). fp8 rows accumulate each 128-dim group apart and scale it in
//           fp32, which is exact.
//   softmax online in base 2; the running max is raised only when a tile exceeds it by more than
//           2^8, otherwise O is not rescaled (the result is the same).
//   P.V     v_mfma_f32_32x32x16_bf16, A = P straight from the Q.K^T accumulators: a lane holds one
//           head and 16 keys, split into two k-steps of 8 slots; B = the same keys' columns read
//           transposed from LDS with ds_read_b64_tr_b16 in the same slot order. An fp8 group
//           scale is folded into P.
// With one split the workgroup writes the bf16 output; with several it writes partials (the
// split's own normalised output in bf16, its max and sum in fp32) that a combine kernel merges.
//
// Picks of -1 (and the padding of a partial last tile) load the row's own latent, which the
// caller has written, and get weight 0: every loaded value is finite.
#include <stddef.h>

#include "dsa_internal.hpp"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int R = 512, PR = 64, KD = R + PR;   // latent, rope, qk width
constexpr int CH = 32;                         // keys per tile
constexpr int HPW = 32;                        // heads per wave
constexpr int kWaves = 4;
constexpr int HPB = HPW * kWaves;              // heads per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxPicks = 4096;                // picks per workgroup (token list in LDS)
constexpr float kLazy = 8.0f;                  // log2 headroom before O is rescaled
constexpr int NB = 3;                          // tiles in the LDS ring

constexpr int kLatRow = R * 2;                 // 1024 bytes: bf16 latent part of a key
constexpr int kLatPitch = kLatRow + 48;        // LDS pitch of a latent row
constexpr int kRopeRow = PR * 2;               // 128 bytes: bf16 rope part of a key
constexpr int kQpePitch = kRopeRow + 16;       // LDS pitch of a head's q_pe (9 bank groups)

template <int LFMT> struct Fmt;
template <> struct Fmt<DSA_FMT_BF16> {
  static constexpr int kRowBytes = KD * 2;     // 1152
  static constexpr int kRopeOff = R * 2;
  static constexpr int kDma = (CH + CH * kRopeRow / 1024) / kWaves;   // DMA instructions per wave per tile
};
template <> struct Fmt<DSA_FMT_FP8> {
  static constexpr int kRowBytes = R + 16 + PR * 2;   // 656: codes, 4 fp32 scales, bf16 rope
  static constexpr int kScaleOff = R;
  static constexpr int kRopeOff = R + 16;
  static constexpr int kDma = 6;               // 4 code, 1 rope, 1 scale instructions per wave
};

// Rope part: piece p of key k in slot p ^ (k & 7).
__device__ __forceinline__ int rope_swz(int k) { return k & 7; }
// fp8 codes in the staging area: piece p of key k in slot p ^ (8 * (k & 1)).
__device__ __forceinline__ int code_swz(int k) { return (k & 1) << 3; }

// LDS layout.
template <int LFMT> struct Smem;
template <> struct Smem<DSA_FMT_BF16> {
  uint8_t lat[NB][CH * kLatPitch];
  uint8_t rope[NB][CH * kRopeRow];
  uint8_t qpe[HPB * kQpePitch];               // the workgroup's q_pe rows
  int tok[kMaxPicks];
  uint32_t valid[kMaxPicks / CH];             // per tile: bit k set if key k is a real pick
};
template <> struct Smem<DSA_FMT_FP8> {
  uint8_t codes[NB][CH * R];                  // raw e4m3 codes
  uint8_t rope[NB][CH * kRopeRow];
  uint8_t scl[NB][kWaves][1024];              // wave w: 16-byte scale records of keys 8w..8w+7 (lanes 0..7)
  uint8_t lat[CH * kLatPitch];                // the current tile's codes as bf16
  float scaleT[4][CH];                        // group scales of the current tile, group-major
  uint8_t qpe[HPB * kQpePitch];               // the workgroup's q_pe rows
  int tok[kMaxPicks];
  uint32_t valid[kMaxPicks / CH];             // per tile: bit k set if key k is a real pick
};

// One 16-byte-per-lane DMA from global memory into LDS: lane l's 16 bytes land at LDS byte
// address m0 + 16 * l (m0 the same in every lane). Issued as assembly so that the compiler does
// not make later LDS reads wait for it (it cannot tell the ring slots apart); completion is
// tracked by hand with wait_vmcnt.
__device__ __forceinline__ void dma16(const void* src, uint32_t m0) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(m0) : "memory");
}

// base + off computed opaquely, so that the compiler keeps later constant offsets in the LDS
// instructions' offset fields instead of re-associating them into per-access additions.
__device__ __forceinline__ uint32_t lds_base(uint32_t base, uint32_t off) {
  uint32_t r;
  asm("v_add_u32 %0, %1, %2" : "=v"(r) : "s"(base), "v"(off));
  return r;
}

__device__ __forceinline__ bf16x8 lds_b128(uint32_t a) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(static_cast<uintptr_t>(a));
}
__device__ __forceinline__ bf16x4 lds_tr16(uint32_t a) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      reinterpret_cast<bf16x4 __attribute__((address_space(3)))*>(static_cast<uintptr_t>(a)));
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p));
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// x *= s for a value held in an AGPR, through one temporary VGPR (the accumulators stay in place
// instead of being copied out as a whole).
__device__ __forceinline__ void scale_agpr(float& x, float s) {
  float tmp;
  asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
               : "+a"(x), "=&v"(tmp) : "v"(s));
}
__device__ __forceinline__ void scale_rows(f32x16& acc, const f32x16& s) {
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    float e = acc[v];
    scale_agpr(e, s[v]);
    acc[v] = e;
  }
}

// 8 e4m3 values (two little-endian words) -> bf16, exactly
__device__ __forceinline__ bf16x8 widen_e4m3(uint32_t w0, uint32_t w1) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  const bf16x4 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  const bf16x4 cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Sink of head h in log2 units of the scaled logits, -inf for none
__device__ __forceinline__ float sink_log2(const float* sink, int h, float scale_log2) {
  if (sink == nullptr) return -__builtin_inff();
  const float v = sink[h];
  return v == -__builtin_inff() ? v : v * scale_log2;
}

template <int LFMT, bool QF8>
__global__ void __launch_bounds__(kThreads, 1)
attend_mfma(DevPlan p, const int32_t* __restrict__ sel, const void* __restrict__ q_nope,
            const void* __restrict__ q_pe, const uint8_t* __restrict__ pool, float scale_log2,
            const float* __restrict__ sink, void* __restrict__ out, uint16_t* __restrict__ part_o,
            float* __restrict__ part_ml, int topk, int H, int n_splits, int log2_ps) {
  __shared__ __attribute__((aligned(16))) Smem<LFMT> sm;
  constexpr bool FP8 = LFMT == DSA_FMT_FP8;
  constexpr int RB = Fmt<LFMT>::kRowBytes;
  constexpr int D = Fmt<LFMT>::kDma;

  const int t = blockIdx.x;
  const int hbase = blockIdx.y * HPB;
  const int split = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const uint32_t sm0 = lds_u32(&sm);
  // The span and this split's picks head the longest chain (span and picks -> page table ->
  // gather) and are requested first; the queries' loads go out behind them, so that the span
  // lookup waits for neither, and the page lookups overlap them.
  const dsa_span span0 = dsa::span_chunk(p.spans, p.n_spans, 0);
  const int per = (topk + n_splits - 1) / n_splits;
  const int k0 = split * per, k1 = min(topk, k0 + per);
  const int npk = max(0, k1 - k0);
  constexpr int kPickPer = kMaxPicks / kThreads;
  int jv[kPickPer];
#pragma unroll
  for (int r = 0; r < kPickPer; ++r) {
    const int i = threadIdx.x + kThreads * r;
    jv[r] = i < npk ? sel[int64_t(t) * topk + k0 + i] : -1;
  }
  asm volatile("" ::: "memory");
  // this wave's 32 queries as the B operand of Q.K^T: head l32, dims 16*ks + 8*g .. +8
  const int head0 = hbase + wave * HPW;
  constexpr int QB = QF8 ? 1 : 2;                     // bytes per query element
  bf16x8 qb[R / 16];
  uint2 qb8[QF8 ? R / 16 : 1];                        // e4m3 queries, widened after the wait below
  // bf16: the wave's 32 query rows are read whole, one 1 KB row per instruction (64 lanes x 16 B,
  // whole cache lines), and reach the lanes that own them through LDS once the picks are staged
  u32x4 qt[QF8 ? 1 : HPW];                            // qt[i]: piece `lane` of head head0 + i
  if constexpr (QF8) {
    const uint8_t* qn = static_cast<const uint8_t*>(q_nope) + (int64_t(t) * H + head0 + l32) * R + 8 * g;
#pragma unroll
    for (int ks = 0; ks < R / 16; ++ks) qb8[ks] = *reinterpret_cast<const uint2*>(qn + 16 * ks);
  } else {
    const uint8_t* qn = static_cast<const uint8_t*>(q_nope) + (int64_t(t) * H + head0) * R * 2 + 16 * lane;
#pragma unroll
    for (int i = 0; i < HPW; ++i) qt[i] = *reinterpret_cast<const u32x4*>(qn + i * R * 2);
  }
  // q_pe of the workgroup's 128 heads, 16-byte pieces (8 per bf16 head, 4 per e4m3 head); it goes
  // to LDS as bf16 (read at its 4 steps per tile) once the token list is built
  constexpr int kPiecesPerHead = PR * QB / 16;
  constexpr int kQpePieces = HPB * kPiecesPerHead / kThreads;
  u32x4 qpe_r[kQpePieces];
  {
    const uint8_t* qp = static_cast<const uint8_t*>(q_pe) + (int64_t(t) * H + hbase) * PR * QB;
#pragma unroll
    for (int i = 0; i < kQpePieces; ++i) {
      const int piece = threadIdx.x + kThreads * i;
      qpe_r[i] = *reinterpret_cast<const u32x4*>(qp + piece * 16);
    }
  }
  // head l32's sink; it waits in LDS for the epilogue rather than hold a register through the loop
  __shared__ float s_sink[HPB];
  const float sk_in = sink_log2(sink, head0 + l32, scale_log2);
  dsa_span sp;
  dsa::row_span_from(span0, p.spans, p.n_spans, t, &sp);
  const int pos = sp.ctx_start + (t - sp.q_start);

  // the picks as pool token indices; a -1 pick (or one outside the row's causal range) is stored
  // as ~own_token: it loads the row's own latent and is masked out of the softmax
  int own;
  {
    int off;
    const int pg = dsa::page_of(p, sp, pos, &off);
    own = (pg << log2_ps) + off;
  }
  // tiles past the split's last real pick are not processed (a causal row below position topk
  // ends in a run of -1 picks)
  int last = -1;
#pragma unroll
  for (int r = 0; r < kPickPer; ++r) {
    const int i = threadIdx.x + kThreads * r;
    if (i < (npk + CH - 1) / CH * CH) {
      int tok = ~own;
      const int j = jv[r];
      if (j >= 0 && j <= pos) {
        int off;
        const int pg = dsa::page_of(p, sp, j, &off);
        tok = (pg << log2_ps) + off;
        last = i;
      }
      sm.tok[i] = tok;
    }
  }
  __shared__ int s_last[kWaves];
  for (int o = 32; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o));
  if (lane == 0) s_last[wave] = last;
#pragma unroll
  for (int i = 0; i < kQpePieces; ++i) {
    const int piece = threadIdx.x + kThreads * i;
    uint8_t* dstq = sm.qpe + (piece / kPiecesPerHead) * kQpePitch;
    if constexpr (QF8) {        // 16 e4m3 values -> 32 bytes of bf16
      const bf16x8 lo = widen_e4m3(qpe_r[i][0], qpe_r[i][1]);
      const bf16x8 hi = widen_e4m3(qpe_r[i][2], qpe_r[i][3]);
      *reinterpret_cast<bf16x8*>(dstq + 32 * (piece % kPiecesPerHead)) = lo;
      *reinterpret_cast<bf16x8*>(dstq + 32 * (piece % kPiecesPerHead) + 16) = hi;
    } else {
      *reinterpret_cast<u32x4*>(dstq + 16 * (piece % kPiecesPerHead)) = qpe_r[i];
    }
  }
  if constexpr (!QF8) {
    // B operand of Q.K^T: lane (l32, g) takes dims 16*ks + 8*g .. +8 of head l32, i.e. piece
    // 2*ks + g of its row. The rows go through this wave's part of the ring buffers (not in use
    // yet) in two rounds of 16 heads, at a pitch of 65 bank groups so that the 16 heads read together
    // fall in distinct banks.
    constexpr int kQtPitch = 1040;
    uint8_t* area = reinterpret_cast<uint8_t*>(&sm) + wave * 16 * kQtPitch;
    static_assert(kWaves * 16 * kQtPitch <= offsetof(Smem<LFMT>, qpe),
                  "query transpose fits in the ring, before the staged q_pe, picks and flags");
#pragma unroll
    for (int r = 0; r < 2; ++r) {
#pragma unroll
      for (int i = 0; i < 16; ++i) *reinterpret_cast<u32x4*>(area + i * kQtPitch + 16 * lane) = qt[16 * r + i];
      if ((l32 >> 4) == r) {
        const uint8_t* row = area + (l32 & 15) * kQtPitch + 16 * g;
#pragma unroll
        for (int ks = 0; ks < R / 16; ++ks) qb[ks] = *reinterpret_cast<const bf16x8*>(row + 32 * ks);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this round's reads are done before the next writes
    }
  }
  __syncthreads();
  int n_tiles = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) n_tiles = max(n_tiles, (s_last[w] + CH) / CH);
  n_tiles = __builtin_amdgcn_readfirstlane(n_tiles);
  for (int c = wave; c < n_tiles; c += kWaves) {
    const uint64_t bits = __builtin_amdgcn_ballot_w64(lane < CH && sm.tok[c * CH + lane] >= 0);
    if (lane == 0) sm.valid[c] = static_cast<uint32_t>(bits);
  }

  // ---- gather of tile c into ring slot b: this wave's D DMA instructions
  // ---- gather of tile c into ring slot b, as kGatherOps DMA instructions per wave: the pool
  // tokens each op needs are read first (gather_keys: op i's token for this lane in tk[i]), then
  // op i issues one DMA (bf16: latent rows of keys 0..7, then the rope parts of all 8; fp8: codes
  // of key pairs, rope, scales)
  constexpr int kGatherOps = D;
  auto tok_at = [&](int idx) {
    const int v = sm.tok[idx];
    return v < 0 ? ~v : v;
  };
  auto gather_keys = [&](int c, int* tk) {
    const int k0 = c * CH + 8 * wave;
    if constexpr (!FP8) {
#pragma unroll
      for (int i = 0; i < 8; ++i) tk[i] = __builtin_amdgcn_readfirstlane(tok_at(k0 + i));
      tk[8] = tok_at(k0 + (lane >> 3));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) tk[i] = tok_at(k0 + 2 * i + (lane >> 5));
      tk[4] = tok_at(k0 + (lane >> 3));
      tk[5] = tok_at(k0 + (lane & 7));
    }
  };
  auto gather_op = [&](int i, const int* tk, int b) {
    if constexpr (!FP8) {
      if (i < 8) {                                  // latent part: one key per instruction
        const int k = 8 * wave + i;
        const uint8_t* src = pool + int64_t(tk[i]) * RB + 16 * lane;
        dma16(src, sm0 + offsetof(Smem<LFMT>, lat) + b * sizeof(sm.lat[0]) + k * kLatPitch);
      } else {                                      // rope part of the 8 keys
        const int k = 8 * wave + (lane >> 3);
        const uint8_t* src = pool + int64_t(tk[8]) * RB + Fmt<LFMT>::kRopeOff + 16 * ((lane & 7) ^ rope_swz(k));
        dma16(src, sm0 + offsetof(Smem<LFMT>, rope) + b * sizeof(sm.rope[0]) + 8 * wave * kRopeRow);
      }
    } else {
      if (i < 4) {                                  // codes: two keys per instruction
        const int k = 8 * wave + 2 * i + (lane >> 5);
        const uint8_t* src = pool + int64_t(tk[i]) * RB + 16 * ((lane & 31) ^ code_swz(k));
        dma16(src, sm0 + offsetof(Smem<LFMT>, codes) + b * sizeof(sm.codes[0]) + (8 * wave + 2 * i) * R);
      } else if (i == 4) {
        const int k = 8 * wave + (lane >> 3);
        const uint8_t* src = pool + int64_t(tk[4]) * RB + Fmt<LFMT>::kRopeOff + 16 * ((lane & 7) ^ rope_swz(k));
        dma16(src, sm0 + offsetof(Smem<LFMT>, rope) + b * sizeof(sm.rope[0]) + 8 * wave * kRopeRow);
      } else {                                      // scale records (lanes 8.. repeat lanes 0..7)
        const uint8_t* src = pool + int64_t(tk[5]) * RB + Fmt<LFMT>::kScaleOff;
        dma16(src, sm0 + offsetof(Smem<LFMT>, scl) + b * sizeof(sm.scl[0]) + wave * sizeof(sm.scl[0][0]));
      }
    }
  };
  constexpr int kTk = FP8 ? 6 : 9;
  auto gather = [&](int c, int b) {
    int tk[kTk];
    gather_keys(c, tk);
#pragma unroll
    for (int i = 0; i < kGatherOps; ++i) gather_op(i, tk, b);
  };

  f32x16 o[R / 32];     // O[head 8*(v/4) + 4*g + v%4][column 32*nt + l32]
#pragma unroll
  for (int i = 0; i < R / 32; ++i) o[i] = f32x16{};
  float m_run = -__builtin_inff();   // running max of head l32 (log2 units)
  float l_run = 0.0f;                // this lane's part of head l32's sum

  // per-lane parts of the LDS operand addresses (tile-independent)
  const uint32_t qk_lane = l32 * kLatPitch + 16 * g;                 // Q.K^T A: key l32, dims 8*g..
  uint32_t rope_lane[PR / 16];                                        // rope k-step u of key l32
#pragma unroll
  for (int u = 0; u < PR / 16; ++u) rope_lane[u] = l32 * kRopeRow + 16 * ((2 * u + g) ^ rope_swz(l32));
  const uint32_t qpe_lane = sm0 + uint32_t(offsetof(Smem<LFMT>, qpe)) + (wave * HPW + l32) * kQpePitch + 16 * g;
  const int j16 = lane & 15, hh = (lane >> 4) & 1;                    // P.V B: first key 4*g + j/4
  const uint32_t pv_lane = (4 * g + (j16 >> 2)) * kLatPitch + 32 * hh + 8 * (j16 & 3);

  wait_vmcnt<0>();   // the queries are in registers: the ring's waits count DMAs only
  if constexpr (QF8) {
#pragma unroll
    for (int ks = 0; ks < R / 16; ++ks) qb[ks] = widen_e4m3(qb8[ks].x, qb8[ks].y);
  }
  if (g == 0) s_sink[wave * HPW + l32] = sk_in;
  // prologue: NB - 1 tiles in flight
#pragma unroll
  for (int c = 0; c < NB - 1; ++c)
    if (c < n_tiles) gather(c, c);
  // bf16: the pool tokens of the next refill are read one iteration ahead (at the end of the
  // previous one), so that its DMAs can go out at once after the tile barrier
  int tk_pre[kTk];
  if constexpr (!FP8) {
    if (NB - 1 < n_tiles) gather_keys(NB - 1, tk_pre);
  }

#pragma clang loop unroll(disable)
  for (int c = 0; c < n_tiles; ++c) {
    const int b = c % NB;
    // this wave's DMAs of tile c are done once at most those of tile c + 1 are outstanding
    if (c + 1 < n_tiles) wait_vmcnt<D * (NB - 2)>(); else wait_vmcnt<0>();
    // tile c visible (each wave waited for its own part of it above); every wave is done with
    // tile c - 1. LDS traffic only: the next tile's gathers stay in flight through the barrier.
    dsa::lds_barrier();
    // Tile c + NB - 1 goes into the slot freed by tile c - 1, all its DMAs at once (bf16 with
    // the pool tokens read one iteration ahead). Each global_load_lds holds the issuing wave for
    // tens of cycles wherever it is placed; here, right after the barrier, the data gets the
    // most time to arrive, and the Q.K^T operand reads that follow run undisturbed.
    const bool refill = c + NB - 1 < n_tiles;
    const int b_next = (b + NB - 1) % NB;
    if constexpr (FP8) {
      if (refill) gather(c + NB - 1, b_next);
    } else {
      if (refill) {
#pragma unroll
        for (int i = 0; i < kGatherOps; ++i) gather_op(i, tk_pre, b_next);
      }
    }

    if constexpr (FP8) {
      // codes -> bf16 latent tile; scale records -> group-major scales
      const int k = threadIdx.x >> 3, j = threadIdx.x & 7;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pc = j + 8 * i;                   // 16 codes
        const u32x4 cw = *reinterpret_cast<const u32x4*>(sm.codes[b] + k * R + 16 * (pc ^ code_swz(k)));
        u32x4 lo, hi;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const bf16x2 x0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[d], 1.0f, false);
          const bf16x2 x1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[d], 1.0f, true);
          const uint32_t w0 = __builtin_bit_cast(uint32_t, x0), w1 = __builtin_bit_cast(uint32_t, x1);
          if (d < 2) { lo[2 * d] = w0; lo[2 * d + 1] = w1; } else { hi[2 * d - 4] = w0; hi[2 * d - 3] = w1; }
        }
        uint8_t* row = sm.lat + k * kLatPitch + 32 * pc;
        *reinterpret_cast<u32x4*>(row) = lo;
        *reinterpret_cast<u32x4*>(row + 16) = hi;
      }
      if (threadIdx.x < 4 * CH) {
        const int gg = threadIdx.x >> 5, kk = threadIdx.x & 31;
        sm.scaleT[gg][kk] = *reinterpret_cast<const float*>(sm.scl[b][kk >> 3] + 16 * (kk & 7) + 4 * gg);
      }
      dsa::lds_barrier();
    }
    // LDS byte addresses of this tile
    uint32_t latb = sm0 + uint32_t(offsetof(Smem<LFMT>, lat));
    if constexpr (!FP8) latb += b * uint32_t(sizeof(sm.lat[0]));
    const uint32_t ropeb = sm0 + uint32_t(offsetof(Smem<LFMT>, rope) + b * sizeof(sm.rope[0]));

    // ---- Q.K^T: 32 keys x 32 heads; lane holds head l32, keys 8*(v/4) + 4*g + v%4.
    // Step u of 36: u < 4 is rope k-step u, else latent k-step u - 4. Operands are read from LDS
    // one window of steps ahead; scheduling barriers keep the register footprint to two windows.
    f32x16 x = f32x16{};
    {
      const uint32_t arow = lds_base(latb, qk_lane);
      auto a_load = [&](int u) -> bf16x8 {
        return u < 4 ? lds_b128(lds_base(ropeb, rope_lane[u])) : lds_b128(arow + 32 * (u - 4));
      };
      // fp8 keeps a second accumulator live, so it reads 2 steps ahead instead of 4
      constexpr int QW = FP8 ? 2 : 4;
      constexpr int NW = 36 / QW;
      bf16x8 A[2][QW];
#pragma unroll
      for (int i = 0; i < QW; ++i) A[0][i] = a_load(i);
      f32x16 acc = f32x16{};
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        if (w + 1 < NW) {
#pragma unroll
          for (int i = 0; i < QW; ++i) A[(w + 1) & 1][i] = a_load(QW * (w + 1) + i);
        }
#pragma unroll
        for (int i = 0; i < QW; ++i) {
          const int u = QW * w + i;
          const bf16x8 qv = u < 4 ? lds_b128(qpe_lane + 32 * u) : qb[u - 4];
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[w & 1][i], qv, acc, 0, 0, 0);
          if constexpr (FP8) {
            // rope (steps 0..3) is unscaled; latent group gg (steps 4+8gg .. 11+8gg) is scaled
            // per key once complete
            if (u == 3) {
              x = acc;
              acc = f32x16{};
            } else if (u > 3 && (u - 3) % 8 == 0) {
              const int gg = (u - 11) / 8;
#pragma unroll
              for (int vq = 0; vq < 4; ++vq) {
                const f32x4 sc = *reinterpret_cast<const f32x4*>(&sm.scaleT[gg][8 * vq + 4 * g]);
#pragma unroll
                for (int r = 0; r < 4; ++r) x[4 * vq + r] = fmaf(sc[r], acc[4 * vq + r], x[4 * vq + r]);
              }
              acc = f32x16{};
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (!FP8) x = acc;
    }

    // ---- online softmax (base 2) for head l32 over this tile's 32 keys (16 here, 16 in lane ^ 32)
    const uint32_t tv = sm.valid[c];
    if (tv != 0xFFFFFFFFu) {                  // keys that are not real picks score -inf
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (!((tv >> (8 * (v >> 2) + 4 * g + (v & 3))) & 1u)) x[v] = -__builtin_inff();
    }
    float mx = x[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mx = fmaxf(mx, x[v]);
    const float mc = fmaxf(mx, __shfl_xor(mx, 32)) * scale_log2;
    float alpha = 1.0f;
    if (mc > m_run + kLazy) {                 // raise the running max; O and the sum rescale
      alpha = m_run != -__builtin_inff() ? __builtin_amdgcn_exp2f(m_run - mc) : 1.0f;
      m_run = mc;
      l_run *= alpha;
    }
    // p = 2^(x * scale - m); with nothing valid yet m is -inf and every x is -inf: p = 0
    const float mneg = m_run != -__builtin_inff() ? -m_run : 0.0f;
    float pv[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      pv[v] = __builtin_amdgcn_exp2f(fmaf(x[v], scale_log2, mneg));
      l_run += pv[v];
    }
    // rescale O rows (heads 8*(v/4) + 4*g + v%4) where their max moved; alpha of head h in lane h
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
      f32x16 av;
#pragma unroll
      for (int v = 0; v < 16; ++v) av[v] = __shfl(alpha, 8 * (v >> 2) + 4 * g + (v & 3));
#pragma unroll
      for (int nt = 0; nt < R / 32; ++nt) scale_rows(o[nt], av);
    }

    // ---- P.V: k-step s holds slots i -> key 16*s + 8*(i/4) + 4*g + i%4 (v = 8*s + i).
    // Transposed B reads: in each 16-lane group, lane j addresses key key0 + j/4, columns
    // c0 + 4*(j%4) .. +3 (8 bytes); the group then holds 4 keys of 16 columns. Step u of 32 is
    // k-step u / 16, column tile u % 16; operands are read one window of 4 steps ahead.
    {
      const uint32_t rbase = lds_base(latb, pv_lane);
      auto b_load = [&](int u, bf16x4* b2) {
        const uint32_t ra = rbase + 16 * (u >> 4) * kLatPitch + 64 * (u & 15);
        b2[0] = lds_tr16(ra);
        b2[1] = lds_tr16(ra + 8 * kLatPitch);
      };
      bf16x4 B[2][4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i) b_load(i, B[0][i]);
      bf16x8 pa;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        if (w + 1 < 8) {
#pragma unroll
          for (int i = 0; i < 4; ++i) b_load(4 * (w + 1) + i, B[(w + 1) & 1][i]);
        }
        const int s = w >> 2;
        if constexpr (FP8) {                          // P times the keys' scales of group w % 4
          const int gg = w & 3;
          const f32x4 s0 = *reinterpret_cast<const f32x4*>(&sm.scaleT[gg][16 * s + 4 * g]);
          const f32x4 s1 = *reinterpret_cast<const f32x4*>(&sm.scaleT[gg][16 * s + 8 + 4 * g]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pa[i] = (__bf16)(pv[8 * s + i] * s0[i]);
            pa[4 + i] = (__bf16)(pv[8 * s + 4 + i] * s1[i]);
          }
        } else if ((w & 3) == 0) {
#pragma unroll
          for (int i = 0; i < 8; ++i) pa[i] = (__bf16)pv[8 * s + i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int nt = 4 * (w & 3) + i;
          // whole-vector shuffle: an element-wise bit cast of shorts into the operand is miscompiled
          const bf16x8 bv = __builtin_shufflevector(B[w & 1][i][0], B[w & 1][i][1], 0, 1, 2, 3, 4, 5, 6, 7);
          o[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, bv, o[nt], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // bf16: the pool tokens of the next refill, one iteration ahead
    if constexpr (!FP8) {
      if (c + NB < n_tiles) gather_keys(c + NB, tk_pre);
    }
  }

  // ---- output: this wave's 32 heads x 512 columns as bf16, normalised by each head's sum (with
  // one split the row's output, else the split's partial). The accumulators hold one column per
  // lane, so the rows go through LDS (the ring is free by now) and leave as 16-byte stores.
  const float lsum = l_run + __shfl_xor(l_run, 32);   // head l32's sum over both lane halves
  const float sk = s_sink[wave * HPW + l32];
  // head l32's output factor: a split's partial is normalised by its own sum; the row's output
  // by sum + sink, taken against the larger of the running max and the sink,
  //   O 2^(m - M) / (l 2^(m - M) + 2^(sink - M)),  M = max(m, sink)
  float inv_h;
  if (n_splits > 1 || sk == -__builtin_inff()) {
    inv_h = lsum > 0.0f ? 1.0f / lsum : 0.0f;
  } else if (m_run == -__builtin_inff()) {
    inv_h = 0.0f;                                     // nothing picked
  } else {
    const float M = fmaxf(m_run, sk);
    const float a = __builtin_amdgcn_exp2f(m_run - M);
    inv_h = a / fmaf(lsum, a, __builtin_amdgcn_exp2f(sk - M));
  }
  const bool out8 = QF8 && n_splits == 1;             // e4m3 rows of R bytes, else bf16 rows
  uint8_t* dst = n_splits == 1 ? static_cast<uint8_t*>(out) + (int64_t(t) * H + head0) * R * QB
                               : reinterpret_cast<uint8_t*>(part_o + ((int64_t(t) * n_splits + split) * H + head0) * R);
  constexpr int kOP = R * 2 + 16;                     // LDS pitch of an output row (bytes)
  static_assert(kWaves * 16 * kOP <= sizeof(Smem<LFMT>) - sizeof(sm.tok) - sizeof(sm.valid),
                "output staging fits in the ring");
  uint8_t* ob = reinterpret_cast<uint8_t*>(&sm) + wave * 16 * kOP;
  wait_vmcnt<0>();
  dsa::lds_barrier();                                 // every wave is done with the ring
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int vv = 0; vv < 8; ++vv) {
      const int v = 8 * half + vv;
      const int hr = 8 * (v >> 2) + 4 * g + (v & 3);  // this lane's head of row v (0..31)
      const float inv = __shfl(inv_h, hr);
      uint8_t* orow = ob + (hr - 16 * half) * kOP;
      if (out8) {
#pragma unroll
        for (int nt = 0; nt < R / 32; ++nt) orow[32 * nt + l32] = uint8_t(dsa::f32_to_e4m3(o[nt][v] * inv));
      } else {
#pragma unroll
        for (int nt = 0; nt < R / 32; ++nt)
          reinterpret_cast<uint16_t*>(orow)[32 * nt + l32] = dsa::f32_to_bf16(o[nt][v] * inv);
      }
    }
    dsa::lds_barrier();
    if (out8) {
      // 16 heads x 32 pieces of 16 columns; instruction i stores heads 16*half + 2i, +1
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int hl = 2 * i + (lane >> 5);
        const u32x4 val = *reinterpret_cast<const u32x4*>(ob + hl * kOP + 16 * (lane & 31));
        *reinterpret_cast<u32x4*>(dst + (16 * half + hl) * R + 16 * (lane & 31)) = val;
      }
    } else {
      // 16 heads x 64 pieces of 8 columns; instruction i stores head 16*half + i, 1 KB
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const u32x4 val = *reinterpret_cast<const u32x4*>(ob + i * kOP + 16 * lane);
        *reinterpret_cast<u32x4*>(dst + ((16 * half + i) * R + 8 * lane) * 2) = val;
      }
    }
    dsa::lds_barrier();
  }
  if (n_splits > 1 && lane < 32) {
    const int64_t prow = (int64_t(t) * n_splits + split) * H + head0;
    part_ml[2 * (prow + lane)] = m_run;
    part_ml[2 * (prow + lane) + 1] = lsum;
  }
}

// out[t][h] = sum_s w_s O_s / (sum_s w_s + 2^(sink - M)), w_s = 2^(m_s - M) l_s, over the S
// splits (O_s is the split's normalised bf16 output; M the largest of the m_s and the sink, whose
// term is absent without one). 128 threads per (row, head), 4 columns each; every partial of a
// thread is loaded before any is used. The output is bf16, or e4m3 for e4m3 queries.
template <int S, bool QF8>
__global__ void __launch_bounds__(256)
attend_combine(const uint16_t* __restrict__ part_o, const float* __restrict__ part_ml,
               const float* __restrict__ sink, float scale_log2, void* __restrict__ out, int H) {
  const int t = blockIdx.x, h = 2 * blockIdx.y + (threadIdx.x >> 7);
  const int c4 = 4 * (threadIdx.x & 127);
  float m[S], l[S];
  uint2 o[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int64_t row = (int64_t(t) * S + s) * H + h;
    const float2 ml = *reinterpret_cast<const float2*>(part_ml + 2 * row);
    m[s] = ml.x;
    l[s] = ml.y;
    o[s] = *reinterpret_cast<const uint2*>(part_o + row * R + c4);
  }
  const float sk = sink_log2(sink, h, scale_log2);
  float M = sk;
#pragma unroll
  for (int s = 0; s < S; ++s) M = fmaxf(M, m[s]);
  float wsum = sk != -__builtin_inff() ? __builtin_amdgcn_exp2f(sk - M) : 0.0f;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const float wgt = l[s] > 0.0f ? __builtin_amdgcn_exp2f(m[s] - M) * l[s] : 0.0f;
    wsum += wgt;
    acc[0] += wgt * __uint_as_float(o[s].x << 16);
    acc[1] += wgt * __uint_as_float(o[s].x & 0xFFFF0000u);
    acc[2] += wgt * __uint_as_float(o[s].y << 16);
    acc[3] += wgt * __uint_as_float(o[s].y & 0xFFFF0000u);
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  const int64_t oi = (int64_t(t) * H + h) * R + c4;
  if constexpr (QF8) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) w |= dsa::f32_to_e4m3(acc[i] * inv) << (8 * i);
    *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(out) + oi) = w;
  } else {
    const uint32_t lo = uint32_t(dsa::f32_to_bf16(acc[0] * inv)) | (uint32_t(dsa::f32_to_bf16(acc[1] * inv)) << 16);
    const uint32_t hi = uint32_t(dsa::f32_to_bf16(acc[2] * inv)) | (uint32_t(dsa::f32_to_bf16(acc[3] * inv)) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + oi) = make_uint2(lo, hi);
  }
}

#ifndef DSA_ATTEND_WG_TARGET
#define DSA_ATTEND_WG_TARGET 256   // workgroups wanted in flight (256 CUs, one workgroup each)
#endif
#ifndef DSA_ATTEND_MIN_PICKS
#define DSA_ATTEND_MIN_PICKS 64    // picks per split at least: partials cost 1 KB per head per split
#endif

int pick_splits(const PlanInfo& in, int H, int topk) {
  // split the picks until the grid covers the chip, keeping DSA_ATTEND_MIN_PICKS per split
  const int base = in.n_rows * (H / HPB);
  int s = 1;
  while (base * s < DSA_ATTEND_WG_TARGET && s * 2 * DSA_ATTEND_MIN_PICKS <= topk && s < 64) s *= 2;
  return s;
}

}  // namespace

bool attend_mfma_supported(const dsa_config& c) {
  const bool pow2 = c.page_size > 0 && (c.page_size & (c.page_size - 1)) == 0;
  return (c.q_fmt == DSA_FMT_BF16 || c.q_fmt == DSA_FMT_FP8) &&
         (c.latent_fmt == DSA_FMT_BF16 || c.latent_fmt == DSA_FMT_FP8) &&
         c.kv_lora_rank == R && c.rope_dim == PR && c.n_heads % HPB == 0 && c.topk <= kMaxPicks && pow2;
}

bool attend_mfma_plan_ok(const DevPlan& p) {
  // pool token indices (page * page_size + offset) must fit a signed 32-bit integer
  return int64_t(p.pool_pages) * p.page_size < (int64_t(1) << 31);
}

int attend_split_count(const PlanInfo& in, int H, int topk);
bool attend_split_supported(const dsa_config& c);

// Packed fp8 latents with bf16 queries go to the 32-head decode kernel whenever the 128-head
// kernel would have to split the picks (too few rows to fill the chip): its partials are a
// quarter the size.
static bool use_split_kernel(const dsa_config& c, const PlanInfo& in) {
  return attend_split_supported(c) && pick_splits(in, c.n_heads, c.topk) > 1;
}

size_t attend_mfma_workspace(const dsa_config& c, const PlanInfo& in) {
  const int s = use_split_kernel(c, in) ? attend_split_count(in, c.n_heads, c.topk)
                                        : pick_splits(in, c.n_heads, c.topk);
  if (s == 1) return 0;
  const size_t rows = size_t(in.n_rows) * s * c.n_heads;
  return ((rows * R * 2 + 255) & ~size_t(255)) + rows * 8;
}

hipError_t launch_attend_combine(int S, bool q8, const uint16_t* part_o, const float* part_ml,
                                 const float* sink, float scale_log2, void* out, int n_rows, int H,
                                 hipStream_t st);
hipError_t launch_attend_split(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                               const int32_t* sel, const void* qn, const void* qp, const void* pool,
                               float sm_scale, const float* sink, void* out, void* ws, int log2_ps,
                               hipStream_t st);

namespace {

template <int LFMT, bool QF8>
hipError_t launch_attend_mfma_t(const dsa_handle* h, const PlanInfo& in, const DevPlan& p,
                                const int32_t* sel, const void* qn, const void* qp, const void* pool,
                                float scale_log2, const float* sink, void* out, uint16_t* part_o,
                                float* part_ml, int s, int log2_ps, hipStream_t st) {
  const dsa_config& c = h->cfg;
  dim3 grid(in.n_rows, c.n_heads / HPB, s);
  hipLaunchKernelGGL((attend_mfma<LFMT, QF8>), grid, dim3(kThreads), 0, st, p, sel, qn, qp,
                     static_cast<const uint8_t*>(pool), scale_log2, sink, out, part_o, part_ml,
                     c.topk, c.n_heads, s, log2_ps);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || s == 1) return e;
  return launch_attend_combine(s, QF8, part_o, part_ml, sink, scale_log2, out, in.n_rows, c.n_heads, st);
}

}  // namespace

// The combine of S split partials per (row, head): S a power of two from 2 to 64.
hipError_t launch_attend_combine(int S, bool q8, const uint16_t* part_o, const float* part_ml,
                                 const float* sink, float scale_log2, void* out, int n_rows, int H,
                                 hipStream_t st) {
  const dim3 cg(n_rows, H / 2);
#define DSA_COMBINE(N)                                                                           \
  case N:                                                                                        \
    if (q8)                                                                                      \
      hipLaunchKernelGGL((attend_combine<N, true>), cg, dim3(256), 0, st, part_o, part_ml, sink, \
                         scale_log2, out, H);                                                    \
    else                                                                                         \
      hipLaunchKernelGGL((attend_combine<N, false>), cg, dim3(256), 0, st, part_o, part_ml, sink, \
                         scale_log2, out, H);                                                    \
    break;
  switch (S) {
    DSA_COMBINE(2)
    DSA_COMBINE(4)
    DSA_COMBINE(8)
    DSA_COMBINE(16)
    DSA_COMBINE(32)
    DSA_COMBINE(64)
    default: return hipErrorInvalidValue;
  }
#undef DSA_COMBINE
  return hipGetLastError();
}

hipError_t launch_attend_mfma(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                              const int32_t* sel, const void* qn, const void* qp, const void* pool,
                              float sm_scale, const float* sink, void* out, void* ws, hipStream_t st) {
  const dsa_config& c = h->cfg;
  int log2_ps = 0;
  while ((1 << log2_ps) < c.page_size) ++log2_ps;
  if (use_split_kernel(c, in))
    return launch_attend_split(h, p, in, sel, qn, qp, pool, sm_scale, sink, out, ws, log2_ps, st);
  const int s = pick_splits(in, c.n_heads, c.topk);
  uint16_t* part_o = nullptr;
  float* part_ml = nullptr;
  if (s > 1) {
    const size_t rows = size_t(in.n_rows) * s * c.n_heads;
    part_o = static_cast<uint16_t*>(ws);
    part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + ((rows * R * 2 + 255) & ~size_t(255)));
  }
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  const bool q8 = c.q_fmt == DSA_FMT_FP8;
  if (c.latent_fmt == DSA_FMT_BF16)
    return q8 ? launch_attend_mfma_t<DSA_FMT_BF16, true>(h, in, p, sel, qn, qp, pool, scale_log2, sink, out, part_o, part_ml, s, log2_ps, st)
              : launch_attend_mfma_t<DSA_FMT_BF16, false>(h, in, p, sel, qn, qp, pool, scale_log2, sink, out, part_o, part_ml, s, log2_ps, st);
  return q8 ? launch_attend_mfma_t<DSA_FMT_FP8, true>(h, in, p, sel, qn, qp, pool, scale_log2, sink, out, part_o, part_ml, s, log2_ps, st)
            : launch_attend_mfma_t<DSA_FMT_FP8, false>(h, in, p, sel, qn, qp, pool, scale_log2, sink, out, part_o, part_ml, s, log2_ps, st);
}
