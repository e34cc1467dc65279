// Absorbed MLA over each row's picked latents on the matrix cores (DSA resource page: attend;
// ttnn.transformer.sparse_sdpa operation line): for row t and head h over picked positions j,
//   logit_j = sm_scale * (q_nope[h] . c_j[0:512] + q_pe[h] . c_j[512:576]),
//   out[h]  = sum_j softmax(logit)_j * c_j[0:512].
// Shapes: 512 + 64 latents (bf16 rows, or packed 656-byte fp8 rows), bf16 queries and output,
// heads a multiple of 64.
//
// A workgroup of 4 waves takes one row, 64 heads and one range of its picks (a split); each wave
// owns 16 heads and all 512 output columns, so waves never exchange softmax state. Picks are
// processed in chunks of 32: their latent rows are gathered into one row-major bf16 LDS tile
// (fp8 codes are converted exactly; their 128-element group scales are kept apart). Per chunk:
//   Q.K^T  v_mfma_f32_16x16x32_bf16 with A = 16 latent rows (LDS), B = the wave's 16 queries
//          (VGPRs), two 16-key tiles; fp8 rows accumulate each 128-dim group apart and scale it
//          in fp32, which is exact;
//   softmax online in base 2; the running max is raised only when a chunk exceeds it by more than
//          2^8, otherwise O is not rescaled (the result is the same);
//   P.V    v_mfma_f32_16x16x32_bf16 with A = P straight from the Q.K^T accumulators: a lane holds
//          one head and keys {4g..4g+3, 16+4g..16+4g+3} (g = lane / 16), and that set is the
//          lane's 8 k-slots; B = the same keys' columns read transposed from the LDS tile with
//          ds_read_b64_tr_b16 in the same slot order. An fp8 group scale is folded into P.
// With one split the workgroup writes the bf16 output; with several it writes fp32 partials
// (max, sum, unnormalised O) that a combine kernel merges.
#include "dsa_internal.hpp"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int R = 512, PR = 64, KD = R + PR;   // latent, rope, qk width
constexpr int CH = 32;                         // picks per chunk
constexpr int LP = KD + 16;                    // LDS pitch of a latent row (bf16 elements)
constexpr int HPB = 64;                        // heads per workgroup
constexpr int HPW = 16;                        // heads per wave
constexpr int kThreads = 256;
constexpr int kMaxPicks = 4096;                // picks per workgroup (token list in LDS)
constexpr float kLazy = 8.0f;                  // log2 headroom before O is rescaled

template <int LFMT> struct Fmt;
template <> struct Fmt<DSA_FMT_BF16> {
  static constexpr int kRowBytes = KD * 2;     // 1152
  static constexpr int kPieces = kRowBytes / 16;
};
template <> struct Fmt<DSA_FMT_FP8> {
  static constexpr int kRowBytes = R + 16 + PR * 2;   // 656
  static constexpr int kPieces = kRowBytes / 16;
};

struct Smem {
  uint16_t lat[CH * LP];     // latent rows of the chunk, bf16
  float gscale[CH][4];       // fp8 group scales of the chunk's rows
  int tok[kMaxPicks];        // pool token index of each pick (-1 = none)
};

// 8 threads gather one key row: thread (k = tid / 8, i = tid % 8) loads 16-byte pieces
// i, i + 8, ... of row k of the chunk.
constexpr int kThreadsPerKey = kThreads / CH;   // 8

template <int LFMT>
__global__ void __launch_bounds__(kThreads, 1)
attend_mfma(DevPlan p, const int32_t* __restrict__ sel, const uint16_t* __restrict__ q_nope,
            const uint16_t* __restrict__ q_pe, const uint8_t* __restrict__ pool, float scale_log2,
            uint16_t* __restrict__ out, float* __restrict__ part_o, float* __restrict__ part_ml,
            int topk, int H, int n_splits, int log2_ps) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
  constexpr int RB = Fmt<LFMT>::kRowBytes;
  constexpr int PPK = Fmt<LFMT>::kPieces;
  constexpr int kLoads = (PPK + kThreadsPerKey - 1) / kThreadsPerKey;

  const int t = blockIdx.x;
  const int hbase = blockIdx.y * HPB;
  const int split = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int s_idx = dsa::find_span(p.spans, p.n_spans, t);
  const dsa_span sp = p.spans[s_idx];
  const int pos = sp.ctx_start + (t - sp.q_start);

  // this wave's 16 queries as the B operand of Q.K^T: head col, dims 32*ks + 8*grp .. +8
  const int grp = lane >> 4, col = lane & 15;
  const int head0 = hbase + wave * HPW;
  bf16x8 qb[18];
  {
    const uint16_t* qn = q_nope + (int64_t(t) * H + head0 + col) * R;
    const uint16_t* qp = q_pe + (int64_t(t) * H + head0 + col) * PR;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) qb[ks] = *reinterpret_cast<const bf16x8*>(qn + 32 * ks + 8 * grp);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) qb[16 + ks] = *reinterpret_cast<const bf16x8*>(qp + 32 * ks + 8 * grp);
  }

  // this split's picks as pool token indices
  const int per = (topk + n_splits - 1) / n_splits;
  const int k0 = split * per, k1 = min(topk, k0 + per);
  const int npk = max(0, k1 - k0);
  for (int i = threadIdx.x; i < npk; i += kThreads) {
    const int j = sel[int64_t(t) * topk + k0 + i];
    int tok = -1;
    if (j >= 0 && j <= pos) {
      int off;
      const int pg = dsa::page_of(p, sp, j, &off);
      tok = (pg << log2_ps) + off;
    }
    sm.tok[i] = tok;
  }

  f32x4 o[32];     // O[head 4*grp + v][column 16*nt + col]
#pragma unroll
  for (int i = 0; i < 32; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();   // running max of head col (log2 units)
  float l_run = 0.0f;                // this lane's part of head col's sum
  __syncthreads();

  const int gk = threadIdx.x / kThreadsPerKey, gi = threadIdx.x % kThreadsPerKey;
  u32x4 gr[kLoads];
  auto gather = [&](int c0) {
    const int idx = c0 + gk;
    const int tok = idx < npk ? sm.tok[idx] : -1;
    const uint8_t* src = pool + int64_t(tok < 0 ? 0 : tok) * RB;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int pk = gi + i * kThreadsPerKey;
      gr[i] = u32x4{0u, 0u, 0u, 0u};
      if (tok >= 0 && pk < PPK) gr[i] = *reinterpret_cast<const u32x4*>(src + 16 * pk);
    }
  };
  auto stage = [&]() {
    uint16_t* row = sm.lat + gk * LP;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int pk = gi + i * kThreadsPerKey;
      if (pk >= PPK) continue;
      if constexpr (LFMT == DSA_FMT_BF16) {
        *reinterpret_cast<u32x4*>(row + 8 * pk) = gr[i];
      } else {
        if (pk < 32) {
          u32x4 lo, hi;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(gr[i][d], 1.0f, false);
            const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(gr[i][d], 1.0f, true);
            const uint32_t wa = __builtin_bit_cast(uint32_t, a), wb = __builtin_bit_cast(uint32_t, b);
            if (d < 2) { lo[2 * d] = wa; lo[2 * d + 1] = wb; } else { hi[2 * (d - 2)] = wa; hi[2 * (d - 2) + 1] = wb; }
          }
          *reinterpret_cast<u32x4*>(row + 16 * pk) = lo;
          *reinterpret_cast<u32x4*>(row + 16 * pk + 8) = hi;
        } else if (pk == 32) {
          sm.gscale[gk][0] = __uint_as_float(gr[i][0]);
          sm.gscale[gk][1] = __uint_as_float(gr[i][1]);
          sm.gscale[gk][2] = __uint_as_float(gr[i][2]);
          sm.gscale[gk][3] = __uint_as_float(gr[i][3]);
        } else {
          *reinterpret_cast<u32x4*>(row + R + 8 * (pk - 33)) = gr[i];
        }
      }
    }
  };

  const int n_chunks = (npk + CH - 1) / CH;
  if (n_chunks > 0) gather(0);
  for (int c = 0; c < n_chunks; ++c) {
    __syncthreads();                       // previous chunk's LDS reads are done
    stage();
    __syncthreads();                       // chunk tile ready
    if (c + 1 < n_chunks) gather((c + 1) * CH);

    // ---- Q.K^T: two 16-key tiles (mt), 16 heads
    constexpr int NG = LFMT == DSA_FMT_FP8 ? 5 : 1;
    f32x4 acc[2][NG];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int g = 0; g < NG; ++g) acc[mt][g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      const int g = LFMT == DSA_FMT_FP8 ? (ks < 16 ? ks / 4 : 4) : 0;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(sm.lat + (16 * mt + col) * LP + 32 * ks + 8 * grp);
        acc[mt][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[ks], acc[mt][g], 0, 0, 0);
      }
    }
    // logits (log2 units): slot i -> key 16*(i/4) + 4*grp + i%4
    float lg[8];
    bool valid[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int mt = i >> 2, v = i & 3;
      const int key = 16 * mt + 4 * grp + v;
      const int idx = c * CH + key;
      valid[i] = idx < npk && sm.tok[idx] >= 0;
      float x;
      if constexpr (LFMT == DSA_FMT_FP8) {
        x = acc[mt][4][v];
        x = fmaf(sm.gscale[key][0], acc[mt][0][v], x);
        x = fmaf(sm.gscale[key][1], acc[mt][1][v], x);
        x = fmaf(sm.gscale[key][2], acc[mt][2][v], x);
        x = fmaf(sm.gscale[key][3], acc[mt][3][v], x);
      } else {
        x = acc[mt][0][v];
      }
      lg[i] = valid[i] ? x * scale_log2 : -__builtin_inff();
    }
    float mc = lg[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mc = fmaxf(mc, lg[i]);
    mc = fmaxf(mc, __shfl_xor(mc, 16));
    mc = fmaxf(mc, __shfl_xor(mc, 32));
    float alpha = 1.0f;
    if (mc > m_run + kLazy) {              // raise the running max; O and sums rescale
      alpha = exp2f(m_run - mc);           // 0 when nothing was accumulated yet
      m_run = mc;
      l_run *= alpha;
    }
    float pv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pv[i] = valid[i] ? exp2f(lg[i] - m_run) : 0.0f;
      l_run += pv[i];
    }
    // rescale O rows (heads 4*grp + v) where the max moved; alpha of head h sits in lane h
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float a = __shfl(alpha, 4 * grp + v);
#pragma unroll
        for (int nt = 0; nt < 32; ++nt) o[nt][v] *= a;
      }
    }
    // P as the A operand, one per column group (fp8: P times the key's group scale)
    constexpr int NPG = LFMT == DSA_FMT_FP8 ? 4 : 1;
    bf16x8 pa[NPG];
#pragma unroll
    for (int g = 0; g < NPG; ++g) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float sc = 1.0f;
        if constexpr (LFMT == DSA_FMT_FP8) sc = sm.gscale[16 * (i >> 2) + 4 * grp + (i & 3)][g];
        pa[g][i] = (__bf16)(pv[i] * sc);
      }
    }
    // ---- P.V: 32 column tiles of 16; B slots follow the A slot keys
    const int li = lane & 15, r = li >> 2, q = li & 3;
    const uint16_t* vrow = sm.lat + (4 * grp + r) * LP + 4 * q;
#pragma unroll
    for (int nt = 0; nt < 32; ++nt) {
      const uint16_t* va = vrow + 16 * nt;
      const bf16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (bf16x4 __attribute__((address_space(3)))*)(va));
      const bf16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (bf16x4 __attribute__((address_space(3)))*)(va + 16 * LP));
      // whole-vector shuffle: an element-wise bit cast of shorts into the operand is miscompiled
      const bf16x8 b = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[LFMT == DSA_FMT_FP8 ? nt / 8 : 0], b, o[nt], 0, 0, 0);
    }
  }

  // ---- head sums over the 4 lane groups
  float lsum = l_run;
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  // O rows of this lane are heads 4*grp + v; their sums and maxima sit in lanes 4*grp + v
  if (n_splits == 1) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float l = __shfl(lsum, 4 * grp + v);
      const float inv = l > 0.0f ? 1.0f / l : 0.0f;
      uint16_t* dst = out + (int64_t(t) * H + head0 + 4 * grp + v) * R + col;
#pragma unroll
      for (int nt = 0; nt < 32; ++nt) dst[16 * nt] = dsa::f32_to_bf16(o[nt][v] * inv);
    }
  } else {
    const int64_t prow = (int64_t(t) * n_splits + split) * H + head0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float* dst = part_o + (prow + 4 * grp + v) * R + col;
#pragma unroll
      for (int nt = 0; nt < 32; ++nt) dst[16 * nt] = o[nt][v];
    }
    if (lane < 16) {
      part_ml[2 * (prow + lane)] = m_run;
      part_ml[2 * (prow + lane) + 1] = lsum;
    }
  }
}

// out[t][h] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s over the splits.
__global__ void __launch_bounds__(256)
attend_combine(const float* __restrict__ part_o, const float* __restrict__ part_ml,
               uint16_t* __restrict__ out, int H, int n_splits) {
  const int t = blockIdx.x, h = blockIdx.y;
  float M = -__builtin_inff();
  for (int s = 0; s < n_splits; ++s) M = fmaxf(M, part_ml[2 * ((int64_t(t) * n_splits + s) * H + h)]);
  float wsum = 0.0f;
  float acc[2] = {0.0f, 0.0f};
  for (int s = 0; s < n_splits; ++s) {
    const int64_t row = (int64_t(t) * n_splits + s) * H + h;
    const float m = part_ml[2 * row], l = part_ml[2 * row + 1];
    if (!(l > 0.0f)) continue;
    const float wgt = exp2f(m - M);
    wsum += wgt * l;
    acc[0] += wgt * part_o[row * R + threadIdx.x];
    acc[1] += wgt * part_o[row * R + 256 + threadIdx.x];
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  uint16_t* dst = out + (int64_t(t) * H + h) * R;
  dst[threadIdx.x] = dsa::f32_to_bf16(acc[0] * inv);
  dst[256 + threadIdx.x] = dsa::f32_to_bf16(acc[1] * inv);
}

#ifndef DSA_ATTEND_WG_TARGET
#define DSA_ATTEND_WG_TARGET 256   // workgroups wanted in flight (256 CUs, one workgroup each)
#endif
#ifndef DSA_ATTEND_MIN_PICKS
#define DSA_ATTEND_MIN_PICKS 128   // picks per split at least: partials cost 2 KB per head per split
#endif

int pick_splits(const PlanInfo& in, int H, int topk) {
  // split the picks until the grid covers the chip, keeping DSA_ATTEND_MIN_PICKS per split
  const int base = in.n_rows * (H / HPB);
  int s = 1;
  while (base * s < DSA_ATTEND_WG_TARGET && s * 2 * DSA_ATTEND_MIN_PICKS <= topk && s < 32) s *= 2;
  return s;
}

}  // namespace

bool attend_mfma_supported(const dsa_config& c) {
  const bool pow2 = c.page_size > 0 && (c.page_size & (c.page_size - 1)) == 0;
  return c.q_fmt == DSA_FMT_BF16 && (c.latent_fmt == DSA_FMT_BF16 || c.latent_fmt == DSA_FMT_FP8) &&
         c.kv_lora_rank == R && c.rope_dim == PR && c.n_heads % HPB == 0 && c.topk <= kMaxPicks && pow2;
}

size_t attend_mfma_workspace(const dsa_config& c, const PlanInfo& in) {
  const int s = pick_splits(in, c.n_heads, c.topk);
  if (s == 1) return 0;
  const size_t rows = size_t(in.n_rows) * s * c.n_heads;
  return ((rows * R * 4 + 255) & ~size_t(255)) + rows * 8;
}

hipError_t launch_attend_mfma(const dsa_handle* h, const DevPlan& p, const PlanInfo& in,
                              const int32_t* sel, const void* qn, const void* qp, const void* pool,
                              float sm_scale, void* out, void* ws, hipStream_t st) {
  const dsa_config& c = h->cfg;
  const int s = pick_splits(in, c.n_heads, c.topk);
  int log2_ps = 0;
  while ((1 << log2_ps) < c.page_size) ++log2_ps;
  float* part_o = nullptr;
  float* part_ml = nullptr;
  if (s > 1) {
    const size_t rows = size_t(in.n_rows) * s * c.n_heads;
    part_o = static_cast<float*>(ws);
    part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + ((rows * R * 4 + 255) & ~size_t(255)));
  }
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  dim3 grid(in.n_rows, c.n_heads / HPB, s);
  const size_t lds = sizeof(Smem);
  if (c.latent_fmt == DSA_FMT_BF16)
    hipLaunchKernelGGL(attend_mfma<DSA_FMT_BF16>, grid, dim3(kThreads), lds, st, p, sel,
                       static_cast<const uint16_t*>(qn), static_cast<const uint16_t*>(qp),
                       static_cast<const uint8_t*>(pool), scale_log2, static_cast<uint16_t*>(out),
                       part_o, part_ml, c.topk, c.n_heads, s, log2_ps);
  else
    hipLaunchKernelGGL(attend_mfma<DSA_FMT_FP8>, grid, dim3(kThreads), lds, st, p, sel,
                       static_cast<const uint16_t*>(qn), static_cast<const uint16_t*>(qp),
                       static_cast<const uint8_t*>(pool), scale_log2, static_cast<uint16_t*>(out),
                       part_o, part_ml, c.topk, c.n_heads, s, log2_ps);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || s == 1) return e;
  hipLaunchKernelGGL(attend_combine, dim3(in.n_rows, c.n_heads), dim3(256), 0, st, part_o, part_ml,
                     static_cast<uint16_t*>(out), c.n_heads, s);
  return hipGetLastError();
}
