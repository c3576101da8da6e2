// Prefill expert FFN: grouped GEMMs on the bf16 matrix cores.
//
// Prefill batches are large enough that each expert's pairs form a real
// matrix (a few hundred rows per expert), so the FFN is a grouped GEMM
// rather than matrix-vector work (the fork README, "Quant types", pairs
// matrix-matrix kernels with prefill).  Per expert: h = silu(X Wg^T) *
// (X Wu^T) with X the expert's gathered token rows, then y = h Wd^T.
//
// Tiles.  A workgroup of eight wavefronts in two groups of four computes
// one row tile of an expert (256 token rows) against two column tiles of 128
// outputs, group g on column tile 2 j + g, with v_mfma_f32_16x16x32_bf16; K
// steps of 64.  Each wavefront owns 64 rows x 128 columns (4 x 8 blocks of
// 16 x 16, 128 accumulators per lane).
//  * The activation tile of a K step (256 rows, bf16) sits in LDS, double
//    buffered, and both groups read it: each activation row is fetched from
//    L2 once per 256 output columns.  The fetch uses whole 128-byte lines
//    (eight lanes per row), two stages before the rows are written to LDS.
//  * Each group dequantises its own weight tile (bf16 = round to nearest even
//    of d * q, exact in fp32 before rounding) into its own double-buffered
//    LDS tile, the blocks' global loads issued two K steps ahead.
//  * A K step of a group is an MFMA phase and a staging phase, each ended by
//    a workgroup barrier, and group 1 runs one phase behind group 0: on every
//    SIMD one wavefront issues matrix instructions while the other stages.
// Gate/up tiles hold 64 gate rows and the 64 up rows of the same
// intermediate indices, so SwiGLU is applied in the accumulator registers.
// An expert's last tile of at most 64 rows (a tail) is computed by all four
// wavefronts of a group on the same rows, each taking two of the eight
// 16-column blocks (a gate block and its up block), so the tail does not
// leave three wavefronts without MFMA work.
//
// Workgroups are dispatched to the 8 XCDs round-robin; the index mapping
// puts all column tiles of one row tile on one XCD so its activation rows
// are read into that XCD's L2 once.
#include <type_traits>

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
// the byte-permute dequantisation of the offset types (WStage FAST): the
// same bits as the conversion path, gate/up 359 -> 349 us at 4096 tokens
// when it was measured on a one-group version of this kernel
constexpr bool kDequantPermute = true;

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
      q4k_block_dm<QT>(row, b, d, m);
      if constexpr (qtype_has_qh(QT)) qh = block_qh<QT>(row, b);
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
// One row tile against column tiles 2 ntp and 2 ntp + 1, as group G (0 or 1)
// of the workgroup: G selects the column tile, the half of the activation
// rows this group stages, and the group's phase (group 1 one behind).
constexpr int kTileRows = 4 * kWaveRows;  // rows of a tile
constexpr int kLdA = kTK + 8;           // LDS row stride of the activation tile (bf16)

struct TileLds {
  __bf16 a[2][kTileRows][kLdA];
  __bf16 b[2][2][kTN][kLdB];  // [group][buffer]
  int pair[kTileRows];
};

// silu(g) u = g u / (1 + e^-g) with the hardware exp2 and reciprocal: a
// few ulp in fp32, far inside the bf16 rounding of h that follows (the
// exact expf and division took several times the instructions in the
// epilogue, which no other wavefront of the SIMD hides)
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g));
}

template <int QT, bool GATEUP, bool SPLIT, int G>
__device__ __forceinline__ void prefill_tile(const FfnParams& p, const __bf16* __restrict__ x, int2 tl, int ntp,
                                        __bf16* __restrict__ hbuf, TileLds& L) {
  constexpr int kUnits = 2;  // half blocks staged per thread and K step: 128 rows x 2 blocks x 2 halves / 256
  const int tid = threadIdx.x, ltid = tid & 255;
  const int lane = tid & (kWave - 1), wave = ltid >> 6, quad = lane >> 4;
  const int e = tl.x, m0 = tl.y;
  const int pbeg = p.offsets[e];
  const int rows = min(kTileRows, p.offsets[e + 1] - pbeg - m0);
  const int slot = p.slot_table[e];
  const int K = GATEUP ? p.H : p.I;
  const int nt_i = 2 * ntp + G;
  const int n0 = GATEUP ? nt_i * (kTN / 2) : nt_i * kTN;
  for (int r = tid; r < kTileRows; r += 512) L.pair[r] = r < rows ? p.sorted_pairs[pbeg + m0 + r] : 0;
  __syncthreads();
  if (slot < 0 || slot >= p.n_slots) {  // both groups see the same expert
    if (tid == 0) atomicCAS(p.err, 0, e + 1);
    if constexpr (GATEUP) {
      for (int idx = ltid; idx < rows * (kTN / 2); idx += 256)
        hbuf[(size_t)(pbeg + m0 + idx / (kTN / 2)) * p.I + n0 + idx % (kTN / 2)] = (__bf16)NAN;
    } else {
      for (int idx = ltid; idx < rows * kTN; idx += 256)
        p.y[(size_t)L.pair[idx / kTN] * p.H + n0 + idx % kTN] = NAN;
    }
    return;
  }
  const int nk = K / kTK;  // even (checked on the host)
  // activation staging: this group's half of the rows, eight lanes per row
  // (16 bytes each), 32 rows per round, four rounds; rows past the tile are
  // neither fetched nor written (their products land in rows never stored)
  const int a_chunk = ltid & 7;
  const __bf16* asrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 128 * G + (ltid >> 3) + 32 * i;
    const int rr = r < rows ? r : 0;
    asrc[i] = (GATEUP ? x + (size_t)(L.pair[rr] / p.k) * p.H : hbuf + (size_t)(pbeg + m0 + rr) * p.I) + 8 * a_chunk;
  }
  bf16x8 areg[2][4];
  const int a_rows = rows - 128 * G - (ltid >> 3);  // this lane's row r is staged when 32 i < a_rows
  auto load_a = [&](bf16x8 (&ar)[4], int kc) {
    const size_t koff = (size_t)min(kc, nk - 1) * kTK;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (32 * i < a_rows) ar[i] = *reinterpret_cast<const bf16x8*>(asrc[i] + koff);
  };
  auto store_a = [&](const bf16x8 (&ar)[4], int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (32 * i < a_rows) *reinterpret_cast<bf16x8*>(&L.a[buf][128 * G + (ltid >> 3) + 32 * i][8 * a_chunk]) = ar[i];
  };
  // weight staging: unit v = ltid * kUnits + u is row v / 4, block (v / 2) % 2, half v % 2
  const int v0 = ltid * kUnits;
  const int brow = v0 >> 2, bblk = (v0 >> 1) & 1;
  const uint8_t* slotp = p.pool + (size_t)slot * p.slot_bytes;
  const uint8_t* wrow;
  if constexpr (GATEUP)
    wrow = slotp + (brow < 64 ? slot_gate_off(QT, p.H, p.I) : slot_up_off(QT, p.H, p.I)) +
           (size_t)(n0 + (brow & 63)) * row_bytes(QT, p.H);
  else
    wrow = slotp + slot_down_off(QT, p.H, p.I) + (size_t)(n0 + brow) * row_bytes(QT, p.I);
  const int scol = 32 * bblk + 16 * (v0 & 1);
  using WS = WStage<QT, kDequantPermute>;
  WS st[2][kUnits];
  auto load_w = [&](WS (&s_)[kUnits], int kc) {
    const int b = 2 * min(kc, nk - 1) + bblk;
#pragma unroll
    for (int u = 0; u < kUnits; ++u) s_[u].load(wrow, b, (v0 + u) & 1);
  };
  auto store_w = [&](const WS (&s_)[kUnits], int buf) {
#pragma unroll
    for (int u = 0; u < kUnits; ++u) s_[u].store(&L.b[G][buf][brow][scol] + 16 * u, (v0 + u) & 1);
  };
  // prologue: activation step 0 (and step 1 for group 1, whose first stage
  // writes step 2), weight step 0; registers for the first two stages
  load_a(areg[0], 0);
  load_w(st[0], 0);
  load_w(st[1], 1);
  store_a(areg[0], 0);
  if constexpr (G == 1) {
    load_a(areg[1], 1);
    store_a(areg[1], 1);
  }
  store_w(st[0], 0);
  load_w(st[0], 2);
  // the stage writing activation step j + G holds it in set (j + G) & 1
  load_a(areg[(1 + G) & 1], 1 + G);
  load_a(areg[(2 + G) & 1], 2 + G);
  __syncthreads();

  f32x4 acc[4][8];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = f32x4{};
  const int row0 = SPLIT ? 0 : kWaveRows * wave;
  const bool active = row0 < rows;
  const int split_mt = (rows + 15) >> 4;  // a tail's 16-row blocks holding rows
  auto phase_end = [] {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  auto mfma_phase = [&](int buf) {
    if (active) {
      __builtin_amdgcn_s_setprio(1);
      const __bf16 (*sa)[kLdA] = L.a[buf];
      const __bf16 (*sb)[kLdB] = L.b[G][buf];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 a[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          a[mt] = *reinterpret_cast<const bf16x8*>(&sa[row0 + 16 * mt + (lane & 15)][32 * ks + 8 * quad]);
        if constexpr (SPLIT) {
          const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(&sb[16 * wave + (lane & 15)][32 * ks + 8 * quad]);
          const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(&sb[16 * (wave + 4) + (lane & 15)][32 * ks + 8 * quad]);
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            if (mt >= split_mt) break;  // 16-row blocks past the tail
            acc[mt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt], b0, acc[mt][0], 0, 0, 0);
            acc[mt][4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt], b1, acc[mt][4], 0, 0, 0);
          }
        } else {
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
                acc[mt][4 * nh + q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt], b[q], acc[mt][4 * nh + q], 0, 0, 0);
          }
        }
      }
      __builtin_amdgcn_s_setprio(0);
    }
    phase_end();
  };
  // stage j (parity P = j & 1): weights of step j into buffer P from st[P]
  // (then st[P] <- step j + 2); activation step j + G into buffer
  // (j + G) & 1 from its register set (then that set <- step j + G + 2)
  auto stage_phase = [&](int j, auto P) {
    constexpr int kP = decltype(P)::value, kS = (kP + G) & 1;
    store_w(st[kP], kP);
    load_w(st[kP], j + 2);
    store_a(areg[kS], kS);
    load_a(areg[kS], j + G + 2);
    phase_end();
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  if constexpr (G == 1) phase_end();
  for (int kc = 0; kc < nk; kc += 2) {
    mfma_phase(0);
    stage_phase(kc + 1, P1{});
    mfma_phase(1);
    stage_phase(kc + 2, P0{});
  }
  if constexpr (G == 0) phase_end();
  if (!active) return;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = row0 + 16 * mt + 4 * quad + r;
      if (m >= rows) continue;
      if constexpr (SPLIT) {
        if constexpr (GATEUP) {
          const float g = acc[mt][0][r], u = acc[mt][4][r];
          hbuf[(size_t)(pbeg + m0 + m) * p.I + n0 + 16 * wave + (lane & 15)] = (__bf16)silu_mul(g, u);
        } else {
          float* yrow = p.y + (size_t)L.pair[m] * p.H + n0 + (lane & 15);
          yrow[16 * wave] = acc[mt][0][r];
          yrow[16 * (wave + 4)] = acc[mt][4][r];
        }
      } else if constexpr (GATEUP) {
        __bf16* hrow = hbuf + (size_t)(pbeg + m0 + m) * p.I + n0 + (lane & 15);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const float g = acc[mt][nt][r], u = acc[mt][nt + 4][r];
          hrow[16 * nt] = (__bf16)silu_mul(g, u);
        }
      } else {
        float* yrow = p.y + (size_t)L.pair[m] * p.H + n0 + (lane & 15);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) yrow[16 * nt] = acc[mt][nt][r];
      }
    }
  }
}

// One launch over both tile lists: the full tiles, then the tails (so the
// tails are dispatched last, into the full tiles' wake).  Each branch is a
// whole tile, so the register allocations never overlap.
template <int QT, bool GATEUP>
__global__ __launch_bounds__(512, 1) void prefill_gemm_kernel(FfnParams p, const __bf16* __restrict__ x,
                                                          const int2* __restrict__ tiles, const int* __restrict__ count,
                                                          int ntn, __bf16* __restrict__ hbuf) {
  __shared__ __attribute__((aligned(16))) TileLds L;
  const int nth = ntn / 2;
  const int j = blockIdx.x / kXcds;
  const int mt_i = kXcds * (j / nth) + (int)(blockIdx.x % kXcds);
  const int ntp = j % nth;
  const int n_big = count[0];
  if (mt_i >= n_big + count[1]) return;
  const bool g1 = threadIdx.x >= 256;
  if (mt_i < n_big) {
    if (g1) prefill_tile<QT, GATEUP, false, 1>(p, x, tiles[mt_i], ntp, hbuf, L);
    else prefill_tile<QT, GATEUP, false, 0>(p, x, tiles[mt_i], ntp, hbuf, L);
  } else {
    if (g1) prefill_tile<QT, GATEUP, true, 1>(p, x, tiles[mt_i], ntp, hbuf, L);
    else prefill_tile<QT, GATEUP, true, 0>(p, x, tiles[mt_i], ntp, hbuf, L);
  }
}

bool prefill_mfma_supported(int H, int I) {
  // column tiles of 128 (down) and 64 (gate/up) in pairs, and an even number
  // of K steps (a multiple of 256 for H and I, as the block layout has)
  return H % (2 * kTN) == 0 && I % (2 * kTN) == 0;
}

// Tried and dropped on the way here (4096-token layer, gate/up): a single
// group of four wavefronts per workgroup, two workgroups per CU, activation
// rows straight into registers (the previous kernel: 354 us against 302
// us), with the MFMA phase at raised priority and the byte-permute
// dequantisation (359 -> 349 us there, both kept here); eight wavefronts on
// 512 rows, slower with one workgroup per CU; the same eight on two column
// tiles in step, without phases (390 us); phases with the activation rows
// in registers rather than LDS (387-392 us); the dequantisation interleaved
// into the MFMAs by scheduling hints (366 us).
static int prefill_max_tiles(size_t P, int E) { return (int)(P / kTileRows) + E + 1; }

size_t prefill_ws_bytes(int T, int k, int I, int E) {
  const size_t P = (size_t)T * k;
  return 256 + ((prefill_max_tiles(P, E) * sizeof(int2) + 255) / 256) * 256 + P * I * sizeof(__bf16);
}

template <bool GATEUP>
static void launch_prefill_gemm(const FfnParams& p, unsigned grid, hipStream_t s, const __bf16* x, const int2* tiles,
                                const int* count, int ntn, __bf16* hbuf) {
#define MOE_PF(Q)                                                                                \
  case Q:                                                                                        \
    launch(prefill_gemm_kernel<Q, GATEUP>, grid, 512, 0, s, p, x, tiles, count, ntn, hbuf);      \
    break;
  switch (p.qtype) {
    MOE_PF(MOE_QTYPE_Q8_0)
    MOE_PF(MOE_QTYPE_Q4_0)
    MOE_PF(MOE_QTYPE_Q4_1)
    MOE_PF(MOE_QTYPE_Q5_0)
    MOE_PF(MOE_QTYPE_Q5_1)
    MOE_PF(MOE_QTYPE_Q4_K)
    MOE_PF(MOE_QTYPE_Q5_K)
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
    launch(prefill_tiles_kernel, 1, 256, 0, s, p.offsets, p.mask, p.E, kTileRows, kWaveRows, tiles, count);
  }
  int rc = check_launch("prefill_tiles_kernel");
  if (rc) return rc;
  const __bf16* xb = (const __bf16*)x;
  {
    KernelTimer timer(ctx, "ffn_gateup", s);
    const int ntn = p.I / (kTN / 2);
    launch_prefill_gemm<true>(p, kXcds * row_groups * (unsigned)(ntn / 2), s, xb, tiles, count, ntn, hbuf);
  }
  if ((rc = check_launch("prefill_gemm_kernel"))) return rc;
  {
    KernelTimer timer(ctx, "ffn_down", s);
    const int ntn = p.H / kTN;
    launch_prefill_gemm<false>(p, kXcds * row_groups * (unsigned)(ntn / 2), s, xb, tiles, count, ntn, hbuf);
  }
  return check_launch("prefill_gemm_kernel");
}

}  // namespace moe
