// Prefill expert FFN: grouped GEMMs on the bf16 matrix cores.
//
// Prefill batches are large enough that each expert's pairs form a real
// matrix (a few hundred rows per expert), so the FFN is a grouped GEMM
// rather than matrix-vector work (the fork README, "Quant types", pairs
// matrix-matrix kernels with prefill).  Per expert: h = silu(X Wg^T) *
// (X Wu^T) with X the expert's gathered token rows, then y = h Wd^T.
//
// Tiles.  A workgroup (4 wavefronts) computes a 256 x 128 output tile of one
// expert with v_mfma_f32_16x16x32_bf16.  Each wavefront owns 64 rows and all
// 128 columns (4 x 8 blocks of 16 x 16, 128 accumulators per lane), so:
//  * activation rows are private to a wavefront and go from global memory
//    (L2) straight into MFMA operand registers, the next K step's loads
//    issued while the current step's MFMAs run;
//  * the weight tile is shared by the four wavefronts through LDS: each
//    thread dequantises one 32-weight block per K step (bf16 = round to
//    nearest even of d * q, exact in fp32 before rounding) into one of two
//    LDS buffers while the MFMAs read the other, one barrier per K step, and
//    the blocks' global loads are issued two K steps ahead.
// Gate/up tiles hold 64 gate rows and the 64 up rows of the same
// intermediate indices, so SwiGLU is applied in the accumulator registers.
//
// Workgroups are dispatched to the 8 XCDs round-robin; the index mapping
// puts all column tiles of one row tile on one XCD so its activation rows
// are read into that XCD's L2 once.
#include "device_common.h"
#include "ffn.h"
#include "route_common.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaveRows = 64;  // rows (pairs) per wavefront
constexpr int kTN = 128;       // output columns per tile
constexpr int kTK = 64;        // K step
constexpr int kLdB = kTK + 8;  // LDS row stride of the weight tile (bf16)
constexpr int kXcds = 8;

// ------------------------------------------------------------ tile list
// One workgroup: for every expert with pairs (and not masked out), its
// tiles of `tile_rows` rows (expert, first row) in expert order, except
// that a last tile of at most `small_rows` rows goes to a second list,
// stored right after the first: count[0] tiles, then count[1] small ones.
__global__ __launch_bounds__(256) void prefill_tiles_kernel(const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ mask, int E, int tile_rows,
                                                            int small_rows, int2* __restrict__ tiles,
                                                            int* __restrict__ count) {
  __shared__ int s_n[kMaxE], s_base[kMaxE], s_ns[kMaxE], s_sbase[kMaxE];
  __shared__ int s_wave[4];
  for (int e = threadIdx.x; e < E; e += 256) {
    const int m = (mask && !mask[e]) ? 0 : offsets[e + 1] - offsets[e];
    const int rem = m % tile_rows;
    const bool small = rem > 0 && rem <= small_rows;
    s_n[e] = m / tile_rows + (rem > small_rows ? 1 : 0);
    s_ns[e] = small ? 1 : 0;
  }
  __syncthreads();
  const int total = block_exclusive_scan<256>(s_n, s_base, E, s_wave);
  __syncthreads();
  const int total_small = block_exclusive_scan<256>(s_ns, s_sbase, E, s_wave);
  for (int e = threadIdx.x; e < E; e += 256) {
    for (int j = 0; j < s_n[e]; ++j) tiles[s_base[e] + j] = make_int2(e, j * tile_rows);
    if (s_ns[e]) tiles[total + s_sbase[e]] = make_int2(e, s_n[e] * tile_rows);
  }
  if (threadIdx.x == 0) {
    count[0] = total;
    count[1] = total_small;
  }
}

// ----------------------------------------------------- weight staging
// 16 consecutive weights (half `h` of a 32-weight block) of a weight row:
// raw codes and scale in registers, then dequantised to bf16 into LDS.
// Q4_0 keeps elements 0..15 in the low nibbles and 16..31 in the high
// nibbles of the block's 16 bytes; Q8_0 half h is bytes 16h..16h+15.
template <int QT, bool FAST = false>
struct WStage {
  uint32_t w[4];
  uint32_t qh;
  float d, m;
  __device__ __forceinline__ void load(const uint8_t* row, int b, int h) {
    const uint8_t* q = block_quants<QT>(row, b) + (QT == MOE_QTYPE_Q8_0 ? 16 * h : 0);
    const uint4 v = *reinterpret_cast<const uint4*>(q);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    if constexpr (qtype_is_k(QT)) {
      q4k_block_dm(row, b, d, m);
      return;
    }
    d = block_scale<QT>(row, b);
    if constexpr (qtype_has_min(QT)) m = block_min<QT>(row, b);
    if constexpr (qtype_has_qh(QT)) qh = block_qh<QT>(row, b);
  }
  // d*q (Q8_0), d*(q-8) (Q4_0), d*(q-16) (Q5_0) as fma(d, u, -OFF*d) with u
  // the unsigned code, or fma(d, u, m) (Q4_1, Q5_1): the product of an
  // 11-bit scale and a code of at most 8 bits is exact in fp32, so the only
  // roundings are the fma's (none without m) and the final one to bf16.
  __device__ __forceinline__ void store(__bf16* dst, int h) const {
    bf16x8 o[2];
    if constexpr (QT == MOE_QTYPE_Q8_0) {
      const float off = -128.0f * d;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t u = w[i] ^ 0x80808080u;  // q + 128 in every byte
#pragma unroll
        for (int j = 0; j < 4; ++j) o[i / 2][(i & 1) * 4 + j] = (__bf16)fmaf(d, (float)((u >> (8 * j)) & 0xFFu), off);
      }
    } else if (FAST && !qtype_has_min(QT)) {
      // code u (at most 5 bits) -> the float 128 + u by placing u in the
      // mantissa of 128.0 (one byte permute), then fma(128 + u, d, -(128 +
      // OFF) d) = d (u - OFF), exact as in the path below: (128 + OFF) d
      // has at most 16 significant bits
      const float c = -(128.0f + qtype_code_off(QT)) * d;
      const int sh = 4 * h;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t nib = (w[i] >> sh) & 0x0F0F0F0Fu;
        if constexpr (qtype_has_qh(QT)) nib |= spread_fifth_bits(qh >> (16 * h + 4 * i));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t bits = __builtin_amdgcn_perm(0x43434343u, nib, 0x04000C0Cu | ((uint32_t)j << 16));
          o[i / 2][(i & 1) * 4 + j] = (__bf16)fmaf(__uint_as_float(bits), d, c);
        }
      }
    } else {
      const float off = qtype_has_min(QT) ? m : -qtype_code_off(QT) * d;
      const int sh = 4 * h;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t nib = (w[i] >> sh) & 0x0F0F0F0Fu;
        if constexpr (qtype_has_qh(QT)) nib |= spread_fifth_bits(qh >> (16 * h + 4 * i));
#pragma unroll
        for (int j = 0; j < 4; ++j) o[i / 2][(i & 1) * 4 + j] = (__bf16)fmaf(d, (float)((nib >> (8 * j)) & 0xFFu), off);
      }
    }
    *reinterpret_cast<bf16x8*>(dst) = o[0];
    *reinterpret_cast<bf16x8*>(dst + 8) = o[1];
  }
};

// ------------------------------------------------------ grouped GEMM
// GATEUP: A = gathered token rows of x (bf16 [T][H]), B = 64 gate + 64 up
// rows, epilogue h = silu(g) * u into hbuf (bf16, grouped order [T*k][I]).
// Down: A = hbuf rows (grouped order), B = 128 rows of Wd, epilogue y
// (fp32, pair order [T*k][H]).  NW wavefronts, 64 rows each.
// One tile (expert e, first row m0; column tile nt_i).  SPLIT: a small
// tile (at most 64 rows, an expert's last rows), where one wavefront of
// rows would leave the others without MFMA work: every wavefront takes the
// same rows and two of the eight 16-column blocks (gate/up: gate block
// `wave` and its up block `wave + 4`, so SwiGLU stays in the wavefront).
// FL bit 0: the MFMA phase of a step at raised wave priority, so of the two
// workgroups on a CU the one with MFMAs to issue is served first while the
// other dequantises; bit 1: WStage's byte-permute dequantisation.
template <int QT, bool GATEUP, int NW, bool SPLIT, int FL = 0>
__device__ __forceinline__ void prefill_tile(const FfnParams& p, const __bf16* __restrict__ x, int2 tl, int nt_i,
                                             __bf16* __restrict__ hbuf, __bf16 (&sB)[2][kTN][kLdB],
                                             int (&s_pair)[kWaveRows * NW]) {
  constexpr int kThreads = 64 * NW, kRows = kWaveRows * NW;
  constexpr int kUnits = 2 * 2 * kTN / kThreads;  // half blocks staged per thread and K step
  const int e = tl.x, m0 = tl.y;
  const int pbeg = p.offsets[e];
  const int rows = min(kRows, p.offsets[e + 1] - pbeg - m0);
  const int slot = p.slot_table[e];
  const int K = GATEUP ? p.H : p.I;
  const int n0 = GATEUP ? nt_i * (kTN / 2) : nt_i * kTN;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6, half = lane >> 5;
  for (int r = tid; r < kRows; r += kThreads) s_pair[r] = r < rows ? p.sorted_pairs[pbeg + m0 + r] : 0;
  __syncthreads();
  if (slot < 0 || slot >= p.n_slots) {
    if (tid == 0) atomicCAS(p.err, 0, e + 1);
    if constexpr (GATEUP) {
      for (int idx = tid; idx < rows * (kTN / 2); idx += kThreads)
        hbuf[(size_t)(pbeg + m0 + idx / (kTN / 2)) * p.I + n0 + idx % (kTN / 2)] = (__bf16)NAN;
    } else {
      for (int idx = tid; idx < rows * kTN; idx += kThreads)
        p.y[(size_t)s_pair[idx / kTN] * p.H + n0 + idx % kTN] = NAN;
    }
    return;
  }
  // activation rows of this lane: MFMA row block mt holds rows 16 mt + lane % 16
  // (rows past the tile's end read row 0; their results are dropped)
  const int quad = lane >> 4;
  const __bf16* arow[4];
  const int row0 = SPLIT ? 0 : kWaveRows * wave;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int m = row0 + 16 * mt + (lane & 15);
    const int mm = m < rows ? m : 0;
    arow[mt] = GATEUP ? x + (size_t)(s_pair[mm] / p.k) * p.H + 8 * quad
                      : hbuf + (size_t)(pbeg + m0 + mm) * p.I + 8 * quad;
  }
  const bool active = row0 < rows;
  // weight staging: unit v = tid * kUnits + u is row v / 4, block (v / 2) % 2, half v % 2
  const int v0 = tid * kUnits;
  const int brow = v0 >> 2, bblk = (v0 >> 1) & 1;
  const uint8_t* slotp = p.pool + (size_t)slot * p.slot_bytes;
  const uint8_t* wrow;
  if constexpr (GATEUP)
    wrow = slotp + (brow < 64 ? slot_gate_off(QT, p.H, p.I) : slot_up_off(QT, p.H, p.I)) +
           (size_t)(n0 + (brow & 63)) * row_bytes(QT, p.H);
  else
    wrow = slotp + slot_down_off(QT, p.H, p.I) + (size_t)(n0 + brow) * row_bytes(QT, p.I);
  const int scol = 32 * bblk + 16 * (v0 & 1);
  __bf16* const sdst0 = &sB[0][brow][scol];
  __bf16* const sdst1 = &sB[1][brow][scol];

  // 4 x 8 blocks of 16 x 16 accumulators (rows 16 mt + 4 (lane / 16) + r, column 16 nt + lane % 16)
  f32x4 acc[4][8];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = f32x4{};
  // activation fragments (row block, 32-wide K half of the step): two
  // register sets, the next step's loads issued at the top of the current
  // step (before the weight prefetch, so waiting for them never waits for
  // a younger load).  Every wavefront loads, even one with no rows in this
  // tile (its rows read row 0): a load under a branch makes the compiler's
  // wait counts assume the path without it.
  bf16x8 a0[4][2], a1[4][2];
  const int nk = K / kTK;  // even (checked on the host)
  auto load_a = [&](bf16x8 (&a)[4][2], int kc) {
    const size_t koff = (size_t)min(kc, nk - 1) * kTK;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) a[mt][ks] = *reinterpret_cast<const bf16x8*>(arow[mt] + koff + 32 * ks);
  };
  using WS = WStage<QT, (FL & 2) != 0>;
  auto load_w = [&](WS (&st)[kUnits], int kc) {
    const int b = 2 * min(kc, nk - 1) + bblk;
#pragma unroll
    for (int u = 0; u < kUnits; ++u) st[u].load(wrow, b, (v0 + u) & 1);
  };
  auto store_w = [&](const WS (&st)[kUnits], __bf16* dst) {
#pragma unroll
    for (int u = 0; u < kUnits; ++u) st[u].store(dst + 16 * u, (v0 + u) & 1);
  };
  load_a(a0, 0);
  WS st0[kUnits], st1[kUnits];
  load_w(st0, 0);
  load_w(st1, 1);
  store_w(st0, sdst0);
  load_w(st0, 2);
  __syncthreads();

  // One K step on buffer `sb` with activations `a`: load the next step's
  // activations into `an`, stage step kc+1 from `nxt` into the other LDS
  // buffer and reload `nxt` with step kc+3, then the MFMAs of step kc.
  // Prefetch indices are clamped to the last step instead of branched on:
  // near the end the repeated loads and the staging into the idle buffer
  // are never read.
  auto step = [&](int kc, const __bf16 (*sb)[kLdB], __bf16* sdst, WS (&nxt)[kUnits],
                  const bf16x8 (&a)[4][2], bf16x8 (&an)[4][2]) {
    load_a(an, kc + 1);
    store_w(nxt, sdst);
    load_w(nxt, kc + 3);
    if constexpr (SPLIT) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(&sb[16 * wave + (lane & 15)][32 * ks + 8 * quad]);
        const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(&sb[16 * (wave + 4) + (lane & 15)][32 * ks + 8 * quad]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          acc[mt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt][ks], b0, acc[mt][0], 0, 0, 0);
          acc[mt][4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt][ks], b1, acc[mt][4], 0, 0, 0);
        }
      }
    } else if (active) {
      if constexpr (FL & 1) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int nh = 0; nh < 2; ++nh) {
          bf16x8 b[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            b[q] = *reinterpret_cast<const bf16x8*>(&sb[16 * (4 * nh + q) + (lane & 15)][32 * ks + 8 * quad]);
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[mt][4 * nh + q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt][ks], b[q], acc[mt][4 * nh + q], 0, 0, 0);
        }
      }
      if constexpr (FL & 1) __builtin_amdgcn_s_setprio(0);
    }
    __syncthreads();
  };
  for (int kc = 0; kc < nk; kc += 2) {
    step(kc, sB[0], sdst1, st1, a0, a1);
    step(kc + 1, sB[1], sdst0, st0, a1, a0);
  }
  if (!active) return;
  if constexpr (SPLIT) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 16 * mt + 4 * quad + r;
        if (m >= rows) continue;
        if constexpr (GATEUP) {
          const float g = acc[mt][0][r], u = acc[mt][4][r];
          hbuf[(size_t)(pbeg + m0 + m) * p.I + n0 + 16 * wave + (lane & 15)] = (__bf16)(g / (1.0f + expf(-g)) * u);
        } else {
          float* yrow = p.y + (size_t)s_pair[m] * p.H + n0 + (lane & 15);
          yrow[16 * wave] = acc[mt][0][r];
          yrow[16 * (wave + 4)] = acc[mt][4][r];
        }
      }
    }
    return;
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = kWaveRows * wave + 16 * mt + 4 * quad + r;
      if (m >= rows) continue;
      if constexpr (GATEUP) {
        __bf16* hrow = hbuf + (size_t)(pbeg + m0 + m) * p.I + n0 + (lane & 15);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const float g = acc[mt][nt][r], u = acc[mt][nt + 4][r];
          hrow[16 * nt] = (__bf16)(g / (1.0f + expf(-g)) * u);
        }
      } else {
        float* yrow = p.y + (size_t)s_pair[m] * p.H + n0 + (lane & 15);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) yrow[16 * nt] = acc[mt][nt][r];
      }
    }
  }
}

// One launch over both lists: the tiles, then the small tiles (so the
// small ones are dispatched last, into the big ones' tail).  Each branch is
// a whole tile, so the two register allocations never overlap.
template <int QT, bool GATEUP, int NW, int FL = 0>
__global__ __launch_bounds__(64 * NW, 2) void prefill_gemm_kernel(FfnParams p, const __bf16* __restrict__ x,
                                                                  const int2* __restrict__ tiles,
                                                                  const int* __restrict__ count, int ntn,
                                                                  __bf16* __restrict__ hbuf) {
  __shared__ __attribute__((aligned(16))) __bf16 sB[2][kTN][kLdB];
  __shared__ int s_pair[kWaveRows * NW];
  const int j = blockIdx.x / kXcds;
  const int mt_i = kXcds * (j / ntn) + (int)(blockIdx.x % kXcds);
  const int nt_i = j % ntn;
  const int n_big = count[0];
  if (mt_i >= n_big + count[1]) return;
  if (mt_i < n_big) prefill_tile<QT, GATEUP, NW, false, FL>(p, x, tiles[mt_i], nt_i, hbuf, sB, s_pair);
  else prefill_tile<QT, GATEUP, NW, true, FL>(p, x, tiles[mt_i], nt_i, hbuf, sB, s_pair);
}

bool prefill_mfma_supported(int H, int I) {
  // column tiles of 128 (down) and 64 (gate/up), and an even number of K steps
  return H % (2 * kTK) == 0 && I % (2 * kTK) == 0 && H % kTN == 0;
}

// Wavefronts per workgroup (64 rows each).  Eight (512 rows, one tile per
// expert of a 4096-token batch) measured slower than four: with one
// workgroup per CU every barrier idles the matrix cores.
constexpr int kPrefillWaves = 4;
// MFMA phase at raised wave priority (bit 0) and the byte-permute
// dequantisation of the offset types (bit 1): bit-identical results,
// gate/up 359 -> 349 us at 4096 tokens.  Tried and dropped: staging one
// row per thread so the LDS writes are free of bank conflicts (the weight
// loads then spread over twice the rows; gate/up 350 -> 374 us), and one
// workgroup per CU with the dequantisation interleaved into the MFMAs by
// scheduling hints (the compiler moved accumulators through AGPRs; 359 ->
// 499 us).
constexpr int kPrefillFlags = 3;
constexpr int kPrefillRows = kWaveRows * kPrefillWaves;

static int prefill_max_tiles(size_t P, int E) { return (int)(P / kPrefillRows) + E + 1; }

size_t prefill_ws_bytes(int T, int k, int I, int E) {
  const size_t P = (size_t)T * k;
  return 256 + ((prefill_max_tiles(P, E) * sizeof(int2) + 255) / 256) * 256 + P * I * sizeof(__bf16);
}

template <bool GATEUP>
static void launch_prefill_gemm(const FfnParams& p, unsigned grid, hipStream_t s, const __bf16* x, const int2* tiles,
                                const int* count, int ntn, __bf16* hbuf) {
#define MOE_PF(Q)                                                                                          \
  case Q:                                                                                                  \
    launch(prefill_gemm_kernel<Q, GATEUP, kPrefillWaves, kPrefillFlags>, grid, 64 * kPrefillWaves, 0, s, p, x, tiles, \
           count, ntn, hbuf);                                                                              \
    break;
  switch (p.qtype) {
    MOE_PF(MOE_QTYPE_Q8_0)
    MOE_PF(MOE_QTYPE_Q4_0)
    MOE_PF(MOE_QTYPE_Q4_1)
    MOE_PF(MOE_QTYPE_Q5_0)
    MOE_PF(MOE_QTYPE_Q5_1)
    MOE_PF(MOE_QTYPE_Q4_K)
    default: break;
  }
#undef MOE_PF
}

int launch_ffn_prefill(moe_ctx* ctx, const FfnParams& p, const void* x, void* ws, hipStream_t s) {
  const size_t P = (size_t)p.T * p.k;
  const int max_tiles = prefill_max_tiles(P, p.E);
  int* count = (int*)ws;
  int2* tiles = (int2*)((char*)ws + 256);
  __bf16* hbuf = (__bf16*)((char*)ws + 256 + ((max_tiles * sizeof(int2) + 255) / 256) * 256);
  const unsigned row_groups = (unsigned)((max_tiles + kXcds - 1) / kXcds);
  {
    KernelTimer timer(ctx, "prefill_tiles", s);
    launch(prefill_tiles_kernel, 1, 256, 0, s, p.offsets, p.mask, p.E, kPrefillRows, kWaveRows, tiles, count);
  }
  int rc = check_launch("prefill_tiles_kernel");
  if (rc) return rc;
  const __bf16* xb = (const __bf16*)x;
  {
    KernelTimer timer(ctx, "ffn_gateup", s);
    const int ntn = p.I / (kTN / 2);
    launch_prefill_gemm<true>(p, kXcds * row_groups * (unsigned)ntn, s, xb, tiles, count, ntn, hbuf);
  }
  if ((rc = check_launch("prefill_gemm_kernel"))) return rc;
  {
    KernelTimer timer(ctx, "ffn_down", s);
    const int ntn = p.H / kTN;
    launch_prefill_gemm<false>(p, kXcds * row_groups * (unsigned)ntn, s, xb, tiles, count, ntn, hbuf);
  }
  return check_launch("prefill_gemm_kernel");
}

}  // namespace moe
