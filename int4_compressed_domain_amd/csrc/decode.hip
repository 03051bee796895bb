// Decode attention directly on the packed cache, one fused kernel.
// [Open-TQ-Metal, arXiv abstract: attention computed on the compressed representation,
//  no intermediate dequantized K/V matrix; the split merge follows the online softmax
//  normalizer cited among its references.]
//
// Work unit u = (sequence b, kv head h); its pages are cut into S context splits, one
// workgroup of NW wavefronts per (u, split). Workgroup order is XCD-aware: MI355X hands
// consecutive workgroups to its 8 XCDs in turn, so all splits of unit u are placed on XCD
// u mod 8, where one L2 holds the unit's query, block-table row and partials.
//
//  prologue  the r = Hq/Hkv queries of head h are rotated into the cache basis with the same
//            fp32 butterfly as the keys (fp16 keys: not rotated), scaled by alpha*log2(e)
//            and a power of two, and split into fp16 hi + lo parts: B-operand columns 0..7
//            hold hi of heads 0..7, columns 8..15 hold lo, so one 16-column MFMA carries
//            ~22 bits of each query. Each wave's first two pages are already loading.
//  page loop each wave takes every NW-th page of the split, two pages per step, streaming
//            later pages into its LDS ring (LDS-DMA) while it computes. Per 16-token page:
//            scores  the K operand is the index bits themselves: (w & 0x000F000F) is the fp16
//                    subnormal u * 2^-24 (exact), so one AND unpacks two indices; the offset
//                    u = c + 8 is removed exactly by starting the MFMA accumulator at -beta,
//                    beta = 8 * 2^-24 * (sum of the 32 query values of the group). One
//                    16x16x32 MFMA per 32-dim group, then times the group's fp16 scale (LUT
//                    keys: the index picks a table value first; fp16 keys: the staged keys
//                    are the A operand);
//            softmax running max/sum per head in the log2 domain, rescaling only when the
//                    max grows;
//            values  the V indices are subnormal A operands too (3- and 2-bit values are
//                    first rebuilt into the 4-bit layout); P' = p * s_V rounded once to
//                    fp16 is the B operand, one 16x16x32 MFMA per group and dim parity for
//                    both pages, and a second one with a constant A removes the offset.
//  epilogue  each wave writes its (o', m, l) into its own ring slots as soon as its loop
//            ends; after one barrier the NW waves merge through LDS (an fp16 tail's slice
//            joins here). With one split the workgroup finishes the head, otherwise it
//            stores its partial (o', m, l), and the last workgroup of the unit to arrive
//            (atomic counter, reset afterwards) merges all splits: every split's (m, l)
//            first, the partials behind them. The result is rotated back (fp32 butterfly,
//            times rho, times sigma) and written.
// Variants: the fused append of each sequence's newest token (knew/vnew), sparse values in
// two passes (SPV), an fp16 tail (hot_k/hot_v).
#include <algorithm>
#include <type_traits>

#include "tq_codec.h"
#include "tq_internal.h"

namespace {

// Subnormal-form K operand: dword of indices of dims e = 0..7 (nibble position e) -> 8
// halves in k-slot order [e0 e4 e1 e5 e2 e6 e3 e7], values u*2^-24 for e0 e4 e2 e6 and
// 16u*2^-24 for e1 e5 e3 e7 (the matching query values are divided by 16).
__device__ __forceinline__ f16x8 unpack_k_sub(uint32_t w) {
  const uint32_t w8 = w >> 8;
  u32x4 r = {w & 0x000F000Fu, w & 0x00F000F0u, w8 & 0x000F000Fu, w8 & 0x00F000F0u};
  return __builtin_bit_cast(f16x8, r);
}

// Geometry of a block and of its staged copy in LDS: [K][V indices][scales]. VB: bits per
// value index; 4-bit values are staged chunk by chunk like the keys, packed 3- and 2-bit
// values as one contiguous copy of their region.
template <int D, int KC, int VB = 4>
struct Cfg {
  static constexpr bool KF16 = KC == TQ_CODEC_FP16;   // fp16 keys
  static constexpr int G = D / 32;
  static constexpr int VC = VB == 4 ? TQ_CODEC_ABSMAX : (VB == 3 ? TQ_CODEC_ABSMAX3 : TQ_CODEC_ABSMAX2);
  static constexpr int BB = tq_block_bytes(D, KC, VC);
  static constexpr int KB = 4 * G;                    // index bytes per lane per page (K or V)
  static constexpr int DMAK = KB >= 16 ? 16 : 4;      // LDS-DMA size for index loads
  static constexpr int NK = KB / DMAK;                // DMAs per index region
  static constexpr int VR = 2 * VB * D;               // V index bytes of a block
  static constexpr int NVP = (VR + 1023) / 1024;      // 16-byte DMAs for packed values
  static constexpr int KREG = KF16 ? 32 * D : 64 * KB;  // staged K bytes (fp16: G runs of 1 KB)
  static constexpr int VOFF = KREG;                   // staged V indices
  static constexpr int SOFF = VOFF + (VB == 4 ? 64 * KB : VR);  // staged scales
  static constexpr int SCB = KF16 ? 32 * G : 64 * G;  // scale bytes (fp16 keys: V scales only)
  static constexpr int NSC = (SCB / 4 + 63) / 64;     // dword DMAs for the scales
  static constexpr int NDMA = (KF16 ? G : NK) + (VB == 4 ? NK : NVP) + NSC;  // vector-memory ops per page
  static constexpr int SLOT = SOFF + SCB;             // LDS bytes of one staged page
  static constexpr int BV = KF16 ? 32 * D : 8 * D;    // block offsets of the V indices
  static constexpr int BS = BV + VR;                  //   and of the scales
  // sparse values, first pass: a page's keys alone ([K indices][K scales], KH bytes) fit
  // half a slot with 4-bit keys, so that pass streams two pages per slot
  static constexpr int KH = KREG + 32 * G;
  static constexpr bool HS = !KF16 && KH <= SLOT / 2 && (SLOT / 2) % 16 == 0;
};

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void*)p;
}

// Buffer loads that write LDS directly (lane i's `n` bytes land at lds + i * n). Issued from
// inline asm so that the only waits for them are the explicit vmcnt waits of the page ring;
// M0 (the LDS base) is set inside the same statement and used by nothing else here.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               ::"v"(voff), "s"(r), "s"(soff), "s"(lds) : "memory");
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dword %0, %1, %2 offen lds"
               ::"v"(voff), "s"(r), "s"(soff), "s"(lds) : "memory");
}

// NB bytes per lane (4, 8, 16 or 32, naturally aligned) into dwords w[0 .. NB/4), with
// non-temporal loads: each page is read once, so it should not displace other data in the
// caches (on MI355X a stream read this way runs ~15% faster than with default loads).
template <int NB>
__device__ __forceinline__ void ld_nt(const uint8_t* p, uint32_t* w) {
  if constexpr (NB == 4) {
    w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
  } else if constexpr (NB == 8) {
    const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    w[0] = x[0];
    w[1] = x[1];
  } else {
#pragma unroll
    for (int c = 0; c < NB / 16; c++) {
      const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + c);
      w[4 * c] = x[0];
      w[4 * c + 1] = x[1];
      w[4 * c + 2] = x[2];
      w[4 * c + 3] = x[3];
    }
  }
}

// Stage one page (one kv head's block) into an LDS slot:
//   [K indices: NK chunks of 64 lanes x DMAK][V indices: same][scales: 16G dwords]
// The buffer descriptor spans exactly this block, so no lane can touch memory outside it.
template <int D, int KC, int VB = 4>
__device__ __forceinline__ void stage_page(const uint8_t* blk, uint32_t base, int lane) {
  using C = Cfg<D, KC, VB>;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)blk, (short)0, C::BB, 0x00020000);
  const uint32_t lo = (uint32_t)lane * C::KB;  // this lane's byte offset inside an index region
  if constexpr (C::KF16) {  // fp16 keys: group g's 1 KB run, 16 bytes per lane
#pragma unroll
    for (int g = 0; g < C::G; g++) dma16(r, (uint32_t)lane * 16, 1024u * g, base + 1024 * g);
  }
#pragma unroll
  for (int c = 0; c < C::NK; c++) {
    if constexpr (C::DMAK == 16) {
      if constexpr (!C::KF16) dma16(r, lo + c * 16, 0u, base + c * 1024);
      if constexpr (VB == 4) dma16(r, lo + c * 16, (uint32_t)C::BV, base + C::VOFF + c * 1024);
    } else {
      if constexpr (!C::KF16) dma4(r, lo + c * 4, 0u, base + c * 256);
      if constexpr (VB == 4) dma4(r, lo + c * 4, (uint32_t)C::BV, base + C::VOFF + c * 256);
    }
  }
  if constexpr (VB < 4) {  // packed values: the region as is, 1 KB per DMA (lane 0 always active)
#pragma unroll
    for (int c = 0; c < C::NVP; c++)
      if (c * 64 + lane < C::VR / 16)
        dma16(r, (uint32_t)(c * 64 + lane) * 16, (uint32_t)C::BV, base + C::VOFF + c * 1024);
  }
#pragma unroll
  for (int c = 0; c < C::NSC; c++)
    if (c * 64 + lane < C::SCB / 4) dma4(r, 4 * (c * 64 + lane), (uint32_t)C::BS, base + C::SOFF + 256 * c);
}

// Sparse values, first pass: the key part of a page ([K][K scales]) alone, into the same slot
// layout as stage_page.
template <int D, int KC, int VB>
struct SplitDma {
  using C = Cfg<D, KC, VB>;
  static constexpr int NSK = C::KF16 ? 0 : (8 * C::G + 63) / 64;  // dword DMAs, K scales
  static constexpr int NK_OPS = (C::KF16 ? C::G : C::NK) + NSK;
};

// The same, compact: K scales right after the K indices (a half slot, see Cfg::HS).
template <int D, int KC, int VB>
__device__ __forceinline__ void stage_kc(const uint8_t* blk, uint32_t base, int lane) {
  using C = Cfg<D, KC, VB>;
  static_assert(C::HS, "compact key staging needs 4-bit keys");
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)blk, (short)0, C::BB, 0x00020000);
  const uint32_t lo = (uint32_t)lane * C::KB;
#pragma unroll
  for (int c = 0; c < C::NK; c++) {
    if constexpr (C::DMAK == 16) dma16(r, lo + c * 16, 0u, base + c * 1024);
    else dma4(r, lo + c * 4, 0u, base + c * 256);
  }
#pragma unroll
  for (int c = 0; c < SplitDma<D, KC, VB>::NSK; c++)
    if (c * 64 + lane < 8 * C::G) dma4(r, 4 * (c * 64 + lane), (uint32_t)C::BS, base + C::KREG + 256 * c);
}

template <int D, int KC, int VB>
__device__ __forceinline__ void stage_k(const uint8_t* blk, uint32_t base, int lane) {
  using C = Cfg<D, KC, VB>;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)blk, (short)0, C::BB, 0x00020000);
  if constexpr (C::KF16) {
#pragma unroll
    for (int g = 0; g < C::G; g++) dma16(r, (uint32_t)lane * 16, 1024u * g, base + 1024 * g);
  } else {
    const uint32_t lo = (uint32_t)lane * C::KB;
#pragma unroll
    for (int c = 0; c < C::NK; c++) {
      if constexpr (C::DMAK == 16) dma16(r, lo + c * 16, 0u, base + c * 1024);
      else dma4(r, lo + c * 4, 0u, base + c * 256);
    }
#pragma unroll
    for (int c = 0; c < SplitDma<D, KC, VB>::NSK; c++)
      if (c * 64 + lane < 8 * C::G) dma4(r, 4 * (c * 64 + lane), (uint32_t)C::BS, base + C::SOFF + 256 * c);
  }
}

// s_waitcnt vmcnt(n * per), n = 0..4 (wave-uniform): every load but the last n*per done.
template <int PER>
__device__ __forceinline__ void wait_all_but(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER) : "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * PER) : "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * PER) : "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * PER) : "memory"); break;
  }
}

// s_waitcnt vmcnt(n) with n a multiple of the per-page DMA count: n = k * NDMA, k = pages
// issued after the one about to be read. The compiler does not track LDS-DMA writes.
template <int NDMA, int K>
__device__ __forceinline__ void wait_pages_in_flight(int k) {
  if constexpr (K == 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    if (k >= K) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(K * NDMA) : "memory");
    else wait_pages_in_flight<NDMA, K - 1>(k);
  }
}

// One butterfly stage across lanes: lane with bit st clear keeps x + partner, the other
// partner - x (its own value is the upper element of the pair).
template <int ST>
__device__ __forceinline__ float bfly(float x, int lane) {
  float y;
  if constexpr (ST < 16) y = dpp_xor<ST>(x, lane);
  else y = __shfl_xor(x, ST, 64);
  return (lane & ST) ? y - x : x + y;
}

// In-wave Walsh-Hadamard butterflies: lane holds V = D/64 values, value k at dim lane + 64k.
// Stages commute, so the in-register strides (64, 128) go first, then lane strides 1..32.
template <int V>
__device__ __forceinline__ void wave_fwht(float (&x)[V], int lane) {
#pragma unroll
  for (int st = 1; st < V; st <<= 1)
#pragma unroll
    for (int k = 0; k < V; k++)
      if (!(k & st)) {
        const float x0 = x[k], x1 = x[k + st];
        x[k] = x0 + x1;
        x[k + st] = x0 - x1;
      }
#pragma unroll
  for (int k = 0; k < V; k++) {
    float y = x[k];
    y = bfly<1>(y, lane);
    y = bfly<2>(y, lane);
    y = bfly<4>(y, lane);
    y = bfly<8>(y, lane);
    y = bfly<16>(y, lane);
    y = bfly<32>(y, lane);
    x[k] = y;
  }
}

// Max over the 64 lanes of a wave (rotations inside rows, then row and half swaps).
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xf, 0xf, true)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xf, 0xf, true)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x122, 0xf, 0xf, true)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x121, 0xf, 0xf, true)));
  return max_xor32(max_xor16(x));
}
__device__ __forceinline__ float wave_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xf, 0xf, true));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xf, 0xf, true));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x122, 0xf, 0xf, true));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x121, 0xf, 0xf, true));
  return sum_xor32(sum_xor16(x));
}

// k-slot of the score MFMA's B operand that holds dim offset e (0..7) of an 8-dim chunk
// (inverse of kslot_dim).
template <int KCODEC>
__device__ __forceinline__ int dim_kslot(int e) {
  if constexpr (KCODEC == TQ_CODEC_ABSMAX) return ((e & 3) << 1) | (e >> 2);
  else if constexpr (KCODEC == TQ_CODEC_FP16) return e;  // fp16 keys: dims in order
  else return (e >> 1) | ((e & 1) << 2);
}

// One query element of dtype dt (fp32, bf16 or fp16), widened exactly.
__device__ __forceinline__ float load_q(const void* q, int dt, int64_t i) {
  if (dt == TQ_F32) return static_cast<const float*>(q)[i];
  if (dt == TQ_BF16) return widen(static_cast<const uint16_t*>(q)[i]);
  return widen(static_cast<const f16*>(q)[i]);
}
// The same in two steps: the element's bits (fp32, or 16 bits zero-extended), then widened.
__device__ __forceinline__ uint32_t load_q_bits(const void* q, int dt, int64_t i) {
  if (dt == TQ_F32) return static_cast<const uint32_t*>(q)[i];
  return static_cast<const uint16_t*>(q)[i];
}
__device__ __forceinline__ float widen_q_bits(uint32_t x, int dt) {
  if (dt == TQ_F32) return __uint_as_float(x);
  if (dt == TQ_BF16) return __uint_as_float(x << 16);
  return (float)__builtin_bit_cast(f16, (uint16_t)x);
}

template <int D, int KCODEC, int VB, int NW, bool SPV>
__global__ __launch_bounds__(64 * NW) void decode_fused(LaunchDecode a) {
  using C = Cfg<D, KCODEC, VB>;
  constexpr int G = C::G, BB = C::BB, NT = 64 * NW, V = D / 64;
  constexpr bool KF16 = C::KF16;
  // ring slots per wave: as many as ~144 KB of LDS holds, at most 8 (NSLOT - 1 pages in
  // flight), or 16 where pages stream through registers (there the ring holds only scale
  // blocks and the merge's scratch, which with small pages needs more than 8 slots)
  constexpr int NSMAX = tq_decode_reg_path(D, KCODEC, VB, SPV) ? 16 : 8;
  constexpr int NSLOT = (147456 / (NW * C::SLOT)) < NSMAX ? (147456 / (NW * C::SLOT)) : NSMAX;
  static_assert(NSLOT >= 3, "ring too small");
  constexpr bool KSUB = (KCODEC == TQ_CODEC_ABSMAX);
  // Register streaming: a page's K and V index dwords are loaded straight into the VGPRs
  // that feed the MFMAs (lane l's bytes of each region are that lane's operand) and its
  // scale block goes to a per-wave LDS slot; other variants stage whole pages in LDS by
  // LDS-DMA. On MI355X the register path streams pages at ~6.2 TB/s, the LDS-DMA path at
  // ~4.5 TB/s (same pages, no compute).
  constexpr bool REG = tq_decode_reg_path(D, KCODEC, VB, SPV);
  constexpr int SW = (C::SCB / 4 + 63) / 64;  // scale dwords per lane of a page (register path)
  constexpr int RG = REG ? G : 1;             // index dwords per lane of a page region
  // register path: pages per step (2 or 4; sparse values' first pass streams the keys
  // alone, half a page's bytes, and packed values' pages are smaller, so those take 4 to
  // keep as many bytes in flight)
  constexpr int PPS = SPV ? 4 : (VB < 4 ? TQ_REG_PPS_PACKED : TQ_REG_PAGES_PER_STEP);
  constexpr int NPR = PPS / 2;                // page pairs per step
  static_assert(!REG || PPS * C::SCB <= C::SLOT, "a page set's scale blocks in one ring slot");
  static_assert(!REG || G <= 4, "register path: D <= 128");
  // register path, V index dwords of a page as loaded: 4-bit values G; packed values the G/2
  // X dwords of the lane's row, then (3-bit) its Z dword (shared by a lane pair at D = 64)
  constexpr int XD = G >= 2 ? G / 2 : 1;
  constexpr int VRG = !REG ? 1 : (VB == 4 ? G : XD + (VB == 3 ? 1 : 0));
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar page loads
  const int jq = lane >> 4, hr = lane & 15, hl = hr & 7;

  // ---- XCD-aware placement: unit u on XCD u mod 8 -----------------------------------------
  const int U = a.B * a.Hkv;
  const int n8 = (U + 7) >> 3;
  const int xcd = blockIdx.x & 7, kk = blockIdx.x >> 3;
  int u = xcd + 8 * (kk % n8);
  const int s = kk / n8;
  if (u >= U) return;
  if (a.order) u = a.order[u];  // longest-first order (see lpt_order_kernel)
  const int b = u / a.Hkv, h = u - b * a.Hkv;
  const int r = a.Hq / a.Hkv;
  const int pps = a.pages_per_split;
  const bool hotwg = a.hot_wg && s >= a.splits;  // one of the unit's a.hot_wg tail workgroups
  const int hwi = hotwg ? s - a.splits : 0;       // (which one)
  const int p0 = hotwg ? 0 : s * pps;

  // ---- the prologue's small loads, issued together with the context length's -----------
  // (one memory round trip): the query bits of this wave's head, the sign bits, and this
  // wave's page ids p0 + wv + NW n. The ids are read up to the split's end in the block
  // table's row, before the sequence's length is known; ids past its last page are never
  // used. They are held across the lanes (page n in lane n % 64 of register n / 64) and read
  // back with v_readlane when issued.
  const int64_t qb = ((int64_t)b * a.Hq + (int64_t)h * r) * D;  // this unit's query elements
  uint32_t qraw[V];  // wave w < r: bits of query head w, dims lane + 64k (widened below)
  if (wv < r) {
#pragma unroll
    for (int k = 0; k < V; k++) qraw[k] = load_q_bits(a.q, a.q_dtype, qb + wv * D + lane + 64 * k);
  }
  const uint32_t sgn_word = tid < D / 32 ? a.sign_bits[tid] : 0u;
  uint32_t qsgn[V];  // sign word of query dim lane + 64k: word 2k + lane / 32 (D >= 64)
#pragma unroll
  for (int k = 0; k < V; k++) qsgn[k] = a.sign_bits[2 * k + (lane >> 5)];
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;
  const int pcap = (hotwg || a.max_ctx == 0) ? 0 : min(p0 + pps, a.max_pages);
  constexpr int PPL = (tq_max_split_pages(NW) / NW + 63) / 64;
  static_assert(PPL <= 4, "page ids of a wave: at most four registers");
  // held in a vector value, not an array: the selection below must stay in registers (as
  // an array it was turned into an indexed access and the ids were moved to LDS, one
  // waited-for load at a time)
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  i32x4 vpid = {0, 0, 0, 0};
#pragma unroll
  for (int k = 0; k < PPL; k++) {
    const int idx = p0 + wv + NW * (lane + 64 * k);
    vpid[k] = idx < pcap ? bt[idx] : 0;
  }
  // Fused append: wave NW - 1 of every workgroup of the unit also loads the unit's new K/V
  // token here (whether its split holds the sequence's last page is known only once the
  // length has arrived); lanes 0..15 take K, 16..31 V, E elements each.
  constexpr int E = CodecCfg<D>::E;
  float ynew[E];
  uint32_t swnew = 0;
  if (!hotwg && a.knew != nullptr && wv == NW - 1 && lane < 32) {
    swnew = lane_signs<D>(a.sign_bits, tq_blk16(lane & 15));
    const int64_t off = ((int64_t)b * a.Hkv + h) * D + tq_blk16(lane & 15) * E;
    const void* src = (lane < 16) ? a.knew : a.vnew;
    if (a.new_dtype == TQ_F32) load_widen<float, E>(static_cast<const float*>(src) + off, ynew);
    else if (a.new_dtype == TQ_BF16) load_widen<uint16_t, E>(static_cast<const uint16_t*>(src) + off, ynew);
    else load_widen<f16, E>(static_cast<const f16*>(src) + off, ynew);
  }
  const int L = a.context_lens[b];
  const int npages = (L + 15) >> 4;
  // Hot/cold: an fp16 tail of Lh recent tokens besides the pool's L. Either every split of
  // the unit takes an equal slice [t0, t0 + tsl) of it after its pages (a unit with a tail
  // and no pool tokens has one split, holding the whole tail), or (a.hot_wg > 0, when the
  // grid has room for it) a.hot_wg more workgroups per unit, split indices a.splits + k,
  // take the tail in pieces of csz tokens and no pages: piece k is [k csz, (k + 1) csz)
  // (the non-empty pieces come first) and publishes partial row ns_cold + k.
  const int Lh = a.hot_k ? min(max(a.hot_lens[b], 0), a.hot_cap) : 0;
  const int ns_cold = (npages + pps - 1) / pps;
  const int csz = a.hot_wg ? (Lh + a.hot_wg - 1) / a.hot_wg : 0;  // tail tokens per piece
  const int nhot = csz > 0 ? (Lh + csz - 1) / csz : 0;             // non-empty pieces
  const int ns = a.hot_wg ? ns_cold + nhot
                          : (ns_cold > 0 ? ns_cold : (Lh > 0 ? 1 : 0));  // partials merged for this unit
  float* outp = a.out + ((int64_t)b * a.Hq + (int64_t)h * r) * D;
  if (ns == 0) {  // empty sequence: zero output, written by split 0
    if (s == 0)
      for (int i = tid; i < r * D; i += NT) outp[i] = 0.0f;
    return;
  }
  if (hotwg ? hwi >= nhot : s >= (a.hot_wg ? ns_cold : ns)) return;
  const int srow = hotwg ? ns_cold + hwi : s;  // this workgroup's partial row
  const int p1 = hotwg ? 0 : min(p0 + pps, npages);
  const int t0 = a.hot_wg ? hwi * csz : (int)((int64_t)Lh * s / ns);
  const int tsl = a.hot_wg ? (hotwg ? min(csz, Lh - t0) : 0) : (int)((int64_t)Lh * (s + 1) / ns) - t0;

  // page ring (per wave) -- reused after the page loop as the merge area
  __shared__ __attribute__((aligned(16))) uint8_t ring[NSLOT][NW][C::SLOT];
  __shared__ __attribute__((aligned(16))) uint8_t tokblk[BB];  // the appended token's codes
  __shared__ float qdown[8];                   // per head: raw score units -> log2 units
  __shared__ float mml[NW][8][2];              // per-wave (m, l), then per-wave weights
  __shared__ float hml[8][2];                  // per head: max M and sum l of the workgroup
  __shared__ int last_flag;
  __shared__ int lead_n;                       // furthest page-loop step reached by a wave
  __shared__ int tok_ready;                    // the appended token is in tokblk
  __shared__ int wskip;                        // sparse values: pages skipped by the workgroup
  __shared__ float mpub[8];                    // sparse values: the unit's maximum so far, per head
  __shared__ uint32_t sgn_s[D / 32];           // sigma bits, read once for the final un-rotation
  // one wave per query head in the rotations: the host admits r <= NW
  static_assert(NW >= 4, "at least four waves");
  // Aliases of the ring: the query operands live in the last slot of every wave until the
  // page loop starts; after the loop, the per-wave results and the final-merge weights.
  static_assert(G * 64 * 8 * 2 <= NW * C::SLOT, "query operands must fit one ring slot row");
  // per-wave results: 8 rows of MOW floats (one per head) in the wave's own ring slots, RPS
  // rows per slot, so that a wave writes them as soon as its page loop ends, while other
  // waves still stream pages through their slots. Rows are padded to D + 4 floats (the rows
  // of one slot then start in different LDS banks) where the ring has room for it.
  constexpr int RING = NSLOT * NW * C::SLOT, SCR = 8 * TQ_MAX_SPLITS * 4 + 8 * (2 * D + TQ_MAX_HOT) * 4;
  constexpr int RPSP = C::SLOT / ((D + 4) * 4) < 8 ? C::SLOT / ((D + 4) * 4) : 8;
  constexpr bool PAD = RPSP > 0 && ((8 + RPSP - 1) / RPSP) * NW * C::SLOT + SCR <= RING;
  constexpr int MOW = PAD ? D + 4 : D;
  constexpr int RPS = C::SLOT / (MOW * 4) < 8 ? C::SLOT / (MOW * 4) : 8;
  constexpr int NRS = RPS > 0 ? (8 + RPS - 1) / RPS : NSLOT + 1;  // slot rows holding them
  static_assert(NRS <= NSLOT, "a wave's results must fit its ring slots");
  constexpr int MEND = NRS * NW * C::SLOT;  // ring bytes below the end of the results
  static_assert(MEND + 8 * TQ_MAX_SPLITS * 4 <= NSLOT * NW * C::SLOT, "merge area must fit the ring");
  static_assert(MEND + 8 * TQ_MAX_SPLITS * 4 + 8 * (2 * D + TQ_MAX_HOT) * 4 <= NSLOT * NW * C::SLOT,
                "the fp16 tail's scratch must fit the ring");
  f16 (*bqs)[64][8] = reinterpret_cast<f16 (*)[64][8]>(&ring[NSLOT - 1][0][0]);
  auto mo = [&](int w, int hd) -> float* {  // row of head hd in wave w's results
    return reinterpret_cast<float*>(&ring[hd / RPS][w][(hd % RPS) * MOW * 4]);
  };
  float (*wsh)[TQ_MAX_SPLITS] = reinterpret_cast<float (*)[TQ_MAX_SPLITS]>(&ring[0][0][0] + MEND);

  // ---- this wave's pages ----------------------------------------------------------------
  const uint8_t* hbase = a.pool + (int64_t)h * BB;
  const int64_t pstride = (int64_t)a.Hkv * BB;
  const int npw = (p1 - p0 - wv + NW - 1) / NW;  // pages of this wave: p0 + wv + NW n, n < npw
  auto page_blk = [&](int n) {  // wave-uniform address of page n's block for head h
    const int id = PPL > 1 ? vpid[(n >> 6) & (PPL - 1)] : vpid[0];
    return hbase + (int64_t)__builtin_amdgcn_readlane(id, n & 63) * pstride;
  };
  // LDS byte address of ring slot k of this wave
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(lds_addr(&ring[0][0][0]));
  auto slot_lds = [&](int k) { return ring_lds + (uint32_t)((k * NW + wv) * C::SLOT); };
  // Fused append: the split holding the sequence's last page also appends its last token
  // (position L - 1) for head h. Wave wc (its token loaded above) quantizes it into tokblk
  // (the block layout, only that token's bytes valid) once the prologue is over, so that the
  // workgroup's start does not wait for it, and raises tok_ready; wave wl, which owns the
  // last page, waits for the flag before it patches the token into that page; wave wc
  // stores the token to the pool after the page loop.
  const bool app = !hotwg && (a.knew != nullptr) && (s == ns_cold - 1);
  const int plast = npages - 1, tnew = (L - 1) & 15;
  const int wc = NW - 1, wl = (plast - p0) % NW;
  int pid_last = 0;  // wave wc: physical id of the last page, for the token's store to the pool
  if (app && wv == wc) pid_last = bt[plast];
  // consume the page ids here, before any page is in flight: otherwise the compiler waits
  // for them (vmcnt(0), i.e. for every in-flight page too) where they are first read
#pragma unroll
  for (int k = 0; k < PPL; k++) asm volatile("" ::"v"(vpid[k]));
  if (tid < D / 32) sgn_s[tid] = sgn_word;  // (read after later barriers: final rotation, tail)
  float qv[V];
  if (wv < r) {  // wave w rotates query head w: sign flip now, butterflies below
#pragma unroll
    for (int k = 0; k < V; k++) {
      const float x = widen_q_bits(qraw[k], a.q_dtype);
      // fp16 keys are in the original basis: the query scores them unrotated
      qv[k] = (!KF16 && ((qsgn[k] >> (lane & 31)) & 1u)) ? -x : x;
    }
  }
  // start streaming this wave's first pages; they land while the queries are prepared
  // sparse values, first pass: NR ring entries per wave, half slots with 4-bit keys
  constexpr int NR = C::HS ? 2 * NSLOT : NSLOT;
  auto k_lds = [&](int n) {  // LDS byte address of the first pass's entry for page n
    if constexpr (C::HS) return slot_lds((n % NR) >> 1) + (uint32_t)(((n % NR) & 1) * (C::SLOT / 2));
    else return slot_lds(n % NSLOT);
  };
  auto k_slot = [&](int n) -> const uint8_t* {
    if constexpr (C::HS) return &ring[(n % NR) >> 1][wv][((n % NR) & 1) * (C::SLOT / 2)];
    else return ring[n % NSLOT][wv];
  };
  auto stage_keys = [&](int n) {
    if constexpr (C::HS) stage_kc<D, KCODEC, VB>(page_blk(n), k_lds(n), lane);
    else stage_k<D, KCODEC, VB>(page_blk(n), k_lds(n), lane);
  };
  auto stage_first = [&]() {
#pragma unroll
    for (int k = 0; k < 2; k++) {
      const int pp = p0 + wv + k * NW;
      if (pp < p1) {
        if constexpr (SPV) stage_keys(k);
        else stage_page<D, KCODEC, VB>(page_blk(k), slot_lds(k), lane);
      }
    }
  };
  // Register path: two page sets of PPS pages, X (step st) and Y (step st + 1), one being
  // computed while the other is in flight. A page n >= npw is a dummy load of one 16-byte
  // line (every lane the same address in the wave's last page), so that every step issues
  // the same loads and the compiler's vmcnt waits stay exact.
  uint32_t xk[PPS][RG], xv[PPS][VRG], xs[PPS][SW], yk[PPS][RG], yv[PPS][VRG], ys[PPS][SW];
  auto ldp = [&](int n, uint32_t (&k)[RG], uint32_t (&v)[VRG], uint32_t (&sw)[SW]) {
    if constexpr (REG) {
      const bool real = n < npw;
      const uint8_t* blk = page_blk(real ? n : npw - 1);
      const uint32_t lo = real ? (uint32_t)lane * C::KB : 0u;
      ld_nt<C::KB>(blk + lo, k);
      if constexpr (VB == 4) {
        ld_nt<C::KB>(blk + C::BV + lo, v);
      } else {
        ld_nt<4 * XD>(blk + C::BV + (real ? (uint32_t)lane * 4 * XD : 0u), v);
        if constexpr (VB == 3) {
          const uint32_t zo = real ? (uint32_t)(G == 2 ? lane >> 1 : lane) * 4 : 0u;
          ld_nt<4>(blk + C::BV + 128 * G + zo, &v[XD]);
        }
      }
#pragma unroll
      for (int i = 0; i < SW; i++) {
        const int dw = real ? min(64 * i + lane, C::SCB / 4 - 1) : 0;
        ld_nt<4>(blk + C::BS + 4 * dw, &sw[i]);
      }
    }
  };
  auto ldstep = [&](int st, uint32_t (&k)[PPS][RG], uint32_t (&v)[PPS][VRG], uint32_t (&sw)[PPS][SW]) {
#pragma unroll
    for (int i = 0; i < PPS; i++) ldp(PPS * st + i, k[i], v[i], sw[i]);
  };
  // sparse values on the register path, first pass: a page's K indices and K scales only
  // (the first half of its scale block), with the same dummy loads past the wave's end
  auto ldk = [&](int n, uint32_t (&k)[RG], uint32_t (&sw)[SW]) {
    if constexpr (REG) {
      const bool real = n < npw;
      const uint8_t* blk = page_blk(real ? n : npw - 1);
      ld_nt<C::KB>(blk + (real ? (uint32_t)lane * C::KB : 0u), k);
#pragma unroll
      for (int i = 0; i < SW; i++) {
        const int dw = real ? min(64 * i + lane, C::SCB / 8 - 1) : 0;
        ld_nt<4>(blk + C::BS + 4 * dw, &sw[i]);
      }
    }
  };
  auto ldkstep = [&](int st, uint32_t (&k)[PPS][RG], uint32_t (&sw)[PPS][SW]) {
#pragma unroll
    for (int i = 0; i < PPS; i++) ldk(PPS * st + i, k[i], sw[i]);
  };
  // Register path: only the first pages are requested before the query is prepared. A
  // wave's loads issue in order, and more than the memory pipeline holds would stall it at
  // the load instructions, holding back the rotation and the barriers behind them (all
  // eight pages up front: the prologue ended 6 to 20 us into the launch instead of ~5).
  constexpr int EARLY = TQ_REG_EARLY < PPS ? TQ_REG_EARLY : PPS;
  if constexpr (REG) {
    if (npw > 0) {
#pragma unroll
      for (int i = 0; i < EARLY; i++) {
        if constexpr (SPV) ldk(i, xk[i], xs[i]);
        else ldp(i, xk[i], xv[i], xs[i]);
      }
    }
  } else {
    stage_first();  // (the query operands go to the last slot, which these loads do not use)
  }

  // ---- prologue: rotate, scale, power-of-two prescale per head ----------------------------
  // Wave w (< r) holds query head w: after the butterflies and scaling it writes the fp16
  // hi part (column w) and lo part (column w + 8) of every dim straight into the B-operand
  // layout: lane 16j + c, k-slot s holds dim 32g + 8j + kslot_dim(s) of group g.
  const float rho = tq_rho(D), qmul = a.attn_scale * TQ_LOG2E;
  if (wv < r) {
    if constexpr (!KF16) wave_fwht<V>(qv, lane);
    float mx = 0.0f;
#pragma unroll
    for (int k = 0; k < V; k++) {
      qv[k] = KF16 ? qv[k] * qmul : (qv[k] * rho) * qmul;
      mx = fmaxf(mx, fabsf(qv[k]));
    }
    mx = wave_max(mx);
    int sh = 0;
    if (mx > 0.0f) sh = min(60, max(-60, 14 - ilogbf(mx)));
    const float up = ldexpf(1.0f, sh);
#pragma unroll
    for (int k = 0; k < V; k++) {
      const int d = lane + 64 * k, g = d >> 5, j = (d >> 3) & 3, sl = dim_kslot<KCODEC>(d & 7);
      const float x = qv[k] * up;
      const f16 hi = (f16)x;
      f16 lo = (f16)(x - (float)hi), hs = hi;
      if (KSUB && (sl & 2)) {  // odd nibble positions carry 16u
        hs = hi * (f16)0.0625f;
        lo = lo * (f16)0.0625f;
      }
      bqs[g][16 * j + wv][sl] = hs;
      bqs[g][16 * j + wv + 8][sl] = lo;
    }
    // scores come out in units of 2^-sh (times 2^24 for the subnormal K form)
    if (lane == 0) qdown[wv] = ldexpf(1.0f, KSUB ? 24 - sh : -sh);
  }
  if (tid == 0) {
    lead_n = 0;
    wskip = 0;
    tok_ready = 0;
  }
  __syncthreads();
  if (app && wv == wc) {  // the appended token, quantized into tokblk
    if (lane < 32) {
      uint32_t un[E];
      f16 scn;
      const int cb = tq_blk16(lane & 15);
      if (KF16 && lane < 16) {
        place_key_f16<D>(tokblk, tnew, cb, ynew);  // fp16 key, no rotation
      } else {
        apply_signs<D>(ynew, swnew);
        if (lane >= 16) codec_vector<D, C::VC>(ynew, cb, un, scn);
        else if (KSUB) codec_vector<D, TQ_CODEC_ABSMAX>(ynew, cb, un, scn);
        else codec_vector<D, TQ_CODEC_LLOYDMAX>(ynew, cb, un, scn);
        place_vector<D, KF16, VB>(tokblk, tnew, cb, lane >= 16, un, scn);
      }
    }
    __hip_atomic_store(&tok_ready, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  // wave wl, before it reads tokblk: the flag is raised by wave wc right after the prologue,
  // which waits for nothing else; the bound only guards against a wait that cannot end
  auto wait_token = [&]() {
    for (int i = 0; i < (1 << 22); i++) {
      if (__hip_atomic_load(&tok_ready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP)) break;
      __builtin_amdgcn_s_sleep(2);
    }
  };
  const bool live = hl < r;
  const bool hiLane = hr < 8;  // lanes 0..7 of a row finish page A of each step, 8..15 page B
  const float down = live ? qdown[hl] : 1.0f;
  // Score operands: column hr holds the hi part (hr < 8) or the lo part (hr >= 8) of the
  // query values of head hr & 7; the two partial scores are added across lanes afterwards.
  f16x8 bq[G];
  float cinit[G];
  // beta = 8 * 2^-24 * (sum of the column's query parts over the group), from one MFMA:
  // A = 8 * 2^-24 in every k-slot (128 * 2^-24 where the B values were divided by 16)
  const f16x8 abeta = __builtin_bit_cast(f16x8, u32x4{0x00080008u, 0x00800080u, 0x00080008u, 0x00800080u});
  const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int g = 0; g < G; g++) {
    bq[g] = *reinterpret_cast<const f16x8*>(&bqs[g][lane][0]);
    if (!live) bq[g] = f16x8{};
    cinit[g] = KSUB ? -__builtin_amdgcn_mfma_f32_16x16x32_f16(abeta, bq[g], zero4, 0, 0, 0)[0] : 0.0f;
  }
  // every wave holds its operands: the last ring slot is free again (the register path
  // never writes that slot: its scale blocks live in the first one)
  if constexpr (!REG) __syncthreads();
  if constexpr (REG) {  // the rest of the first two steps' pages
    if (npw > 0) {
      if constexpr (SPV) {
#pragma unroll
        for (int i = EARLY; i < PPS; i++) ldk(i, xk[i], xs[i]);
        ldkstep(1, yk, ys);
      } else {
#pragma unroll
        for (int i = EARLY; i < PPS; i++) ldp(i, xk[i], xv[i], xs[i]);
        ldstep(1, yk, yv, ys);
      }
    }
  }
  uint32_t tlo[4] = {0, 0, 0, 0}, thi[4] = {0, 0, 0, 0};
  if constexpr (KCODEC == TQ_CODEC_LLOYDMAX) {
    const uint16_t lb[16] = TQ_LUT16_BITS;
#pragma unroll
    for (int i = 0; i < 16; i++) {
      tlo[i >> 2] |= (uint32_t)(lb[i] & 0xffu) << (8 * (i & 3));
      thi[i >> 2] |= (uint32_t)(lb[i] >> 8) << (8 * (i & 3));
    }
  }
  // V operands are subnormal fp16 too: (w & 0x000F000F) = u * 2^-24 (even dims) and
  // (w & 0x00F000F0) = 16u * 2^-24 (odd dims). The offset u = c + 8 is removed pair by pair
  // by a second MFMA whose A operand is the constant -8 * 2^-24 (-128 * 2^-24 for odd dims):
  // it adds -8 * 2^-24 * sum_t P'_t to every row, so the accumulator always holds the signed
  // sum and never the offset-biased one.
  // (3- and 2-bit values: offsets 4 and 2, so -4 or -2 * 2^-24 and -64 or -32 * 2^-24)
  constexpr uint32_t CEV = VB == 4 ? 0x80088008u : (VB == 3 ? 0x80048004u : 0x80028002u);
  constexpr uint32_t COD = VB == 4 ? 0x80808080u : (VB == 3 ? 0x80408040u : 0x80208020u);
  u32x4 ce4 = {CEV, CEV, CEV, CEV};
  u32x4 co4 = {COD, COD, COD, COD};
  asm("" : "+v"(ce4), "+v"(co4));  // keep the constant operands in VGPRs
  const f16x8 ceven = __builtin_bit_cast(f16x8, ce4), codd = __builtin_bit_cast(f16x8, co4);
  const int ltail = L & 15;
  const int ptail = ltail ? npages - 1 : -1;  // the sequence's partial last page, if any

  // ---- page loop: two pages per step ----------------------------------------------------
  // Wave wv takes pages p0 + wv + NW n, n = 0, 1, ...; step i handles n = 2i (page A) and
  // 2i + 1 (page B). Scores of both pages come from the MFMAs in every lane; then lanes with
  // hr < 8 finish page A and lanes with hr >= 8 page B (same head hr & 7), so the softmax and
  // P' work is not duplicated, and one K = 32 MFMA per group accumulates both pages.
  f32x4 acc[2 * G];
#pragma unroll
  for (int t = 0; t < 2 * G; t++) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // m_run: running max of the raw scores (shared by lanes hr and hr ^ 8); nmd = -m_run * down
  float m_run = -INFINITY, nmd = INFINITY, l_run = 0.0f;

  auto load_idx = [&](const uint8_t* slot, uint32_t (&w)[G], int region) {  // region 0: K, 1: V
    if constexpr (VB < 4) {
      if (region) {
        // packed values back to the 4-bit layout's dwords w[g] (indices in the low 3 or 2
        // bits of each nibble): X dword g/2 of this lane's row, shifted by 2*(g%2), and for
        // 3 bits Z dword (lane*G + g)/4, shifted by (lane*G + g)%4, into bit 2
        const uint8_t* vr = slot + C::VOFF;
        uint32_t X[G >= 2 ? G / 2 : 1];
        if constexpr (G == 2) {
          X[0] = *reinterpret_cast<const uint32_t*>(vr + lane * 4);
        } else if constexpr (G == 4) {
          const u32x2 x2 = *reinterpret_cast<const u32x2*>(vr + lane * 8);
          X[0] = x2[0]; X[1] = x2[1];
        } else {
          const u32x4 x4 = *reinterpret_cast<const u32x4*>(vr + lane * 16);
          X[0] = x4[0]; X[1] = x4[1]; X[2] = x4[2]; X[3] = x4[3];
        }
#pragma unroll
        for (int g = 0; g < G; g++) w[g] = (X[g >> 1] >> (2 * (g & 1))) & 0x33333333u;
        if constexpr (VB == 3) {
          const uint8_t* zr = vr + 128 * G;
          if constexpr (G == 2) {
            const uint32_t z = *reinterpret_cast<const uint32_t*>(zr + (lane >> 1) * 4) >> (2 * (lane & 1));
#pragma unroll
            for (int g = 0; g < G; g++) w[g] |= ((z >> g) & 0x11111111u) << 2;
          } else {
            uint32_t Z[G / 4];
            if constexpr (G == 4) {
              Z[0] = *reinterpret_cast<const uint32_t*>(zr + lane * 4);
            } else {
              const u32x2 z2 = *reinterpret_cast<const u32x2*>(zr + lane * 8);
              Z[0] = z2[0]; Z[1] = z2[1];
            }
#pragma unroll
            for (int g = 0; g < G; g++) w[g] |= ((Z[g >> 2] >> (g & 3)) & 0x11111111u) << 2;
          }
        }
        return;
      }
    }
#pragma unroll
    for (int c = 0; c < C::NK; c++) {
      if constexpr (C::DMAK == 16) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(slot + (region ? C::VOFF : 0) + c * 1024 + lane * 16);
        w[4 * c] = x[0]; w[4 * c + 1] = x[1]; w[4 * c + 2] = x[2]; w[4 * c + 3] = x[3];
      } else {
        w[c] = *reinterpret_cast<const uint32_t*>(slot + (region ? C::VOFF : 0) + c * 256 + lane * 4);
      }
    }
  };
  auto load_scales = [&](const uint8_t* slot, uint32_t (&st)[2 * G], int region,
                         int soff = C::SOFF) {  // region 0: K, 1: V
    const uint32_t* sw = reinterpret_cast<const uint32_t*>(slot + soff);
    const int roff = KF16 ? 0 : region * 8 * G;  // fp16 keys: only V scales are staged
#pragma unroll
    for (int i = 0; i < 2 * G; i += 4) {  // fp16 pairs: tokens 4jq..4jq+3, groups 0..G-1
      const u32x4 x = *reinterpret_cast<const u32x4*>(&sw[roff + 2 * G * jq + i]);
      st[i] = x[0]; st[i + 1] = x[1]; st[i + 2] = x[2]; st[i + 3] = x[3];
    }
  };
  auto kop = [&](uint32_t w) -> f16x8 {
    if constexpr (KSUB) return unpack_k_sub(w);
    else return unpack_k_lut(w, tlo, thi);
  };
  auto scale_of = [](const uint32_t (&st)[2 * G], int e, int g) {
    return (float)as_h2(st[(e * G + g) >> 1])[(e * G + g) & 1];
  };
  // one page's partial scores in every lane (column hr: hi or lo part), from its K index
  // dwords and the K scales at sbase + kso
  auto scores_w = [&](const uint32_t (&kw)[G], const uint8_t* sbase, int kso, float (&sc)[4]) {
    uint32_t kst[2 * G];
    load_scales(sbase, kst, 0, kso);
#pragma unroll
    for (int e = 0; e < 4; e++) sc[e] = 0.0f;
#pragma unroll
    for (int g = 0; g < G; g++) {
      const f32x4 ci = {cinit[g], cinit[g], cinit[g], cinit[g]};
      const f32x4 c = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop(kw[g]), bq[g], ci, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; e++) sc[e] = __builtin_fmaf(scale_of(kst, e, g), c[e], sc[e]);
    }
  };
  // the same for a page staged in an LDS slot (K scales at slot + kso)
  auto scores = [&](const uint8_t* slot, float (&sc)[4], int kso = C::SOFF) {
    if constexpr (KF16) {  // fp16 keys are the A operand as staged; one accumulator
      f32x4 c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int g = 0; g < G; g++)
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(*reinterpret_cast<const f16x8*>(slot + 1024 * g + lane * 16),
                                                    bq[g], c, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; e++) sc[e] = c[e];
      return;
    }
    uint32_t kw[G];
    load_idx(slot, kw, 0);
    scores_w(kw, slot, kso, sc);
  };

  // One step over pages A and B from their partial scores (sA, sB); vidx(vwA, vwB) fetches
  // their V index dwords, the V scales are read from svA / svB + svoff (the lane's own page).
  auto step_core = [&](const float (&sA)[4], const float (&sB)[4], auto&& vidx, const uint8_t* svA,
                       const uint8_t* svB, int svoff, int pa, int pb) {
    float sc[4];
    // own page's hi (or lo) part plus the partner lane's part of the same page
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const float own = hiLane ? sA[e] : sB[e];
      const float sup = hiLane ? sB[e] : sA[e];
      sc[e] = own + dpp_ror8(sup);
    }
    uint32_t vst[2 * G];  // V scales of this lane's page
    load_scales(hiLane ? svA : svB, vst, 1, svoff);
    if (pa == ptail || pb == ptail || pb >= p1) {  // wave-uniform: a partial or missing page
      const int pm = hiLane ? pa : pb;
      const int lim = (pm >= p1) ? 0 : (pm == ptail ? ltail : 16);
#pragma unroll
      for (int e = 0; e < 4; e++)
        if (4 * jq + e >= lim) {
          sc[e] = -INFINITY;
#pragma unroll
          for (int g = 0; g < G; g += 2) vst[(e * G + g) >> 1] = 0u;  // slot may hold garbage
        }
    }
    float cm = vmax3(sc[0], sc[1], vmax(sc[2], sc[3]));
    cm = max_xor16(cm);
    cm = max_xor32(cm);
    cm = vmax(cm, dpp_ror8(cm));
    if (__any(cm > m_run)) {
      const float mn = fmaxf(m_run, cm);
      const float f = __builtin_amdgcn_exp2f((m_run - mn) * down);  // 2^-inf = 0
      l_run *= f;
#pragma unroll
      for (int t = 0; t < 2 * G; t++) acc[t] *= f;
      m_run = mn;
      nmd = -mn * down;
    }
    float pr[4];
#pragma unroll
    for (int e = 0; e < 4; e++) pr[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e], down, nmd));
    l_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);

    uint32_t vwA[G], vwB[G];
    vidx(vwA, vwB);
    auto vsc = [&](int e, int g) { return (float)as_h2(vst[(e * G + g) >> 1])[(e * G + g) & 1]; };
#pragma unroll
    for (int g = 0; g < G; g++) {
      // P' = p * s_V of this lane's page, rounded once to fp16, k-slot token order 0 2 1 3;
      // k-slots 0..3 of the operand are page A, 4..7 page B (from the partner lane)
      const f16x4 own = {(f16)__builtin_fmaf(pr[0], vsc(0, g), 0.0f), (f16)__builtin_fmaf(pr[2], vsc(2, g), 0.0f),
                         (f16)__builtin_fmaf(pr[1], vsc(1, g), 0.0f), (f16)__builtin_fmaf(pr[3], vsc(3, g), 0.0f)};
      const u32x2 o2 = __builtin_bit_cast(u32x2, own);
      const uint32_t x0 = __builtin_amdgcn_mov_dpp(o2[0], 0x128, 0xf, 0xf, true);
      const uint32_t x1 = __builtin_amdgcn_mov_dpp(o2[1], 0x128, 0xf, 0xf, true);
      const f16x8 P = __builtin_bit_cast(f16x8, u32x4{o2[0], o2[1], x0, x1});
      const uint32_t a = vwA[g], a8 = a >> 8, bw = vwB[g], b8 = bw >> 8;
      const f16x8 Ae = __builtin_bit_cast(f16x8, u32x4{a & 0x000F000Fu, a8 & 0x000F000Fu, bw & 0x000F000Fu, b8 & 0x000F000Fu});
      const f16x8 Ao = __builtin_bit_cast(f16x8, u32x4{a & 0x00F000F0u, a8 & 0x00F000F0u, bw & 0x00F000F0u, b8 & 0x00F000F0u});
      acc[2 * g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ae, P, acc[2 * g], 0, 0, 0);
      acc[2 * g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ceven, P, acc[2 * g], 0, 0, 0);
      acc[2 * g + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ao, P, acc[2 * g + 1], 0, 0, 0);
      acc[2 * g + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(codd, P, acc[2 * g + 1], 0, 0, 0);
    }
  };
  // a step over two pages staged in LDS slots
  auto step = [&](const uint8_t* slotA, const uint8_t* slotB, int pa, int pb) {
    float sA[4], sB[4];
    scores(slotA, sA);
    scores(slotB, sB);
    step_core(sA, sB, [&](uint32_t (&wa)[G], uint32_t (&wb)[G]) {
      load_idx(slotA, wa, 1);
      load_idx(slotB, wb, 1);
    }, slotA, slotB, C::SOFF, pa, pb);
  };
  // Register path, one step over PPS pages held in registers: pairs (0, 1), (2, 3), ...,
  // each finished as in step_core (lanes with hr < 8 the first page of a pair, the others
  // the second); the running max is updated once per step. ss: the pages' scale blocks in
  // LDS, pa0: the global number of page 0 (pages pa0 + NW i).
  // a register page's V index dwords in the 4-bit layout (packed values unpacked as
  // load_idx does for a staged page: X dword g/2 shifted by 2(g%2), Z bits into bit 2)
  auto vregs = [&](const uint32_t (&raw)[VRG], uint32_t (&w)[G]) {
    if constexpr (VB == 4 || !REG) {
#pragma unroll
      for (int g = 0; g < G; g++) w[g] = raw[VB == 4 ? g : 0];
    } else {
#pragma unroll
      for (int g = 0; g < G; g++) w[g] = (raw[g >> 1] >> (2 * (g & 1))) & 0x33333333u;
      if constexpr (VB == 3) {
        const uint32_t z = raw[XD] >> (G == 2 ? 2 * (lane & 1) : 0);
#pragma unroll
        for (int g = 0; g < G; g++) w[g] |= ((z >> g) & 0x11111111u) << 2;
      }
    }
  };
  auto stepN = [&](const uint32_t (&kk)[PPS][RG], const uint32_t (&vv)[PPS][VRG], const uint8_t* ss,
                   const int (&pg)[PPS]) {
    if constexpr (REG) {
      float s4[PPS][4];
#pragma unroll
      for (int i = 0; i < PPS; i++) scores_w(kk[i], ss + i * C::SCB, 0, s4[i]);
      float sc[NPR][4];
      uint32_t vst[NPR][2 * G];  // V scales of this lane's page of each pair
#pragma unroll
      for (int j = 0; j < NPR; j++) {
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const float own = hiLane ? s4[2 * j][e] : s4[2 * j + 1][e];
          const float sup = hiLane ? s4[2 * j + 1][e] : s4[2 * j][e];
          sc[j][e] = own + dpp_ror8(sup);
        }
        load_scales(ss + (hiLane ? 2 * j : 2 * j + 1) * C::SCB, vst[j], 1, 0);
      }
      bool edge = false;  // wave-uniform: a partial or missing page in the step
#pragma unroll
      for (int i = 0; i < PPS; i++) edge |= pg[i] >= p1 || pg[i] == ptail;
      if (edge) {
#pragma unroll
        for (int j = 0; j < NPR; j++) {
          const int pm = hiLane ? pg[2 * j] : pg[2 * j + 1];
          const int lim = (pm >= p1) ? 0 : (pm == ptail ? ltail : 16);
#pragma unroll
          for (int e = 0; e < 4; e++)
            if (4 * jq + e >= lim) {
              sc[j][e] = -INFINITY;
#pragma unroll
              for (int g = 0; g < G; g += 2) vst[j][(e * G + g) >> 1] = 0u;  // may hold garbage
            }
        }
      }
      float cm = vmax3(sc[0][0], sc[0][1], vmax(sc[0][2], sc[0][3]));
#pragma unroll
      for (int j = 1; j < NPR; j++) cm = vmax3(cm, vmax3(sc[j][0], sc[j][1], sc[j][2]), sc[j][3]);
      cm = max_xor16(cm);
      cm = max_xor32(cm);
      cm = vmax(cm, dpp_ror8(cm));
      if (__any(cm > m_run)) {
        const float mn = fmaxf(m_run, cm);
        const float f = __builtin_amdgcn_exp2f((m_run - mn) * down);  // 2^-inf = 0
        l_run *= f;
#pragma unroll
        for (int t = 0; t < 2 * G; t++) acc[t] *= f;
        m_run = mn;
        nmd = -mn * down;
      }
      float pr[NPR][4];
#pragma unroll
      for (int j = 0; j < NPR; j++)
#pragma unroll
        for (int e = 0; e < 4; e++) pr[j][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[j][e], down, nmd));
#pragma unroll
      for (int j = 0; j < NPR; j++) l_run += (pr[j][0] + pr[j][1]) + (pr[j][2] + pr[j][3]);
#pragma unroll
      for (int j = 0; j < NPR; j++) {
        auto vsc = [&](int e, int g) { return (float)as_h2(vst[j][(e * G + g) >> 1])[(e * G + g) & 1]; };
        uint32_t wA[G], wB[G];
        vregs(vv[2 * j], wA);
        vregs(vv[2 * j + 1], wB);
#pragma unroll
        for (int g = 0; g < G; g++) {
          // P' as in step_core: this lane's page in k-slots 0..3 (own) or 4..7 (partner)
          const f16x4 own = {(f16)__builtin_fmaf(pr[j][0], vsc(0, g), 0.0f), (f16)__builtin_fmaf(pr[j][2], vsc(2, g), 0.0f),
                             (f16)__builtin_fmaf(pr[j][1], vsc(1, g), 0.0f), (f16)__builtin_fmaf(pr[j][3], vsc(3, g), 0.0f)};
          const u32x2 o2 = __builtin_bit_cast(u32x2, own);
          const uint32_t x0 = __builtin_amdgcn_mov_dpp(o2[0], 0x128, 0xf, 0xf, true);
          const uint32_t x1 = __builtin_amdgcn_mov_dpp(o2[1], 0x128, 0xf, 0xf, true);
          const f16x8 P = __builtin_bit_cast(f16x8, u32x4{o2[0], o2[1], x0, x1});
          const uint32_t a = wA[g], a8 = a >> 8, bw = wB[g], b8 = bw >> 8;
          const f16x8 Ae = __builtin_bit_cast(f16x8, u32x4{a & 0x000F000Fu, a8 & 0x000F000Fu, bw & 0x000F000Fu, b8 & 0x000F000Fu});
          const f16x8 Ao = __builtin_bit_cast(f16x8, u32x4{a & 0x00F000F0u, a8 & 0x00F000F0u, bw & 0x00F000F0u, b8 & 0x00F000F0u});
          acc[2 * g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ae, P, acc[2 * g], 0, 0, 0);
          acc[2 * g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ceven, P, acc[2 * g], 0, 0, 0);
          acc[2 * g + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ao, P, acc[2 * g + 1], 0, 0, 0);
          acc[2 * g + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(codd, P, acc[2 * g + 1], 0, 0, 0);
        }
      }
    }
  };

  // ---- sparse values, pass 1: keys only. The running max and sum of every token are kept
  // as in the dense loop (no values), and each page's largest score per head goes to pmreg:
  // entry 8n + h (wave page n, head h) in lane (8n + h) % 64 of register n / 8, which after
  // the reductions below is lane 16 ((n / 2) % 4) + hr of the step that scores page n.
  constexpr int NPM = TQ_SPARSE_PAGES_PER_WAVE / 8;  // registers of page maxima
  static_assert(NPM == 4, "four registers of page maxima");
  // (a vector value, written by selects: as an array its updates became an indexed store
  // that the compiler placed in scratch memory)
  f32x4 pmreg = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  int nskip = 0;  // pages of this wave whose values were skipped
  auto kstep = [&](int na_, const uint8_t* slotA, const uint8_t* slotB, int pa, int pb) {
    float sc[4], sA[4], sB[4];
    constexpr int kso = C::HS ? C::KREG : C::SOFF;  // where the first pass put the K scales
    scores(slotA, sA, kso);
    scores(slotB, sB, kso);
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const float own = hiLane ? sA[e] : sB[e];
      const float sup = hiLane ? sB[e] : sA[e];
      sc[e] = own + dpp_ror8(sup);
    }
    if (pa == ptail || pb == ptail || pb >= p1) {  // wave-uniform: a partial or missing page
      const int pm = hiLane ? pa : pb;
      const int lim = (pm >= p1) ? 0 : (pm == ptail ? ltail : 16);
#pragma unroll
      for (int e = 0; e < 4; e++)
        if (4 * jq + e >= lim) sc[e] = -INFINITY;
    }
    float pmx = vmax3(sc[0], sc[1], vmax(sc[2], sc[3]));
    pmx = max_xor16(pmx);
    pmx = max_xor32(pmx);  // this lane's page (A if hiLane), head hl: its largest score
    const int kreg = na_ >> 3, kq = (na_ >> 1) & 3;
#pragma unroll
    for (int k = 0; k < NPM; k++)
      pmreg[k] = (k == kreg && jq == kq) ? pmx : pmreg[k];
    const float cm = vmax(pmx, dpp_ror8(pmx));  // both pages
    if (__any(cm > m_run)) {
      const float mn = fmaxf(m_run, cm);
      l_run *= __builtin_amdgcn_exp2f((m_run - mn) * down);  // 2^-inf = 0
      m_run = mn;
      nmd = -mn * down;
    }
#pragma unroll
    for (int e = 0; e < 4; e++) l_run += __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e], down, nmd));
  };

  // Copy the appended token's bytes (indices and scales of token tnew) from tokblk into a
  // block: the pool (to_lds = false), or the staged LDS copy of the last page, whose index
  // regions are stored chunk by chunk as the page loads wrote them (see stage_page). With
  // keys_only, only its key bytes and K scales, into a key-only staged copy of sparse
  // values' first pass whose K scales start at kso (stage_k, stage_kc).
  auto copy_token = [&](uint8_t* dst, bool to_lds, bool keys_only = false, int kso = C::SOFF) {
    constexpr int G_ = D / 32, KB = C::KB, DM = C::DMAK;
    // staged position of a 4-bit index byte w of an index region (page loads write each
    // region chunk by chunk: chunk w / DM of every lane, lane after lane)
    auto staged = [&](int w) {
      const int l = w / KB, wb = w % KB;
      return (wb / DM) * (64 * DM) + l * DM + (wb % DM);
    };
    auto at = [&](int o) {  // block offset -> offset in dst
      if (!to_lds) return o;
      if (o < C::BV) return KF16 ? o : staged(o);  // keys (fp16 keys are staged as stored)
      if (o < C::BS) return VB == 4 ? C::VOFF + staged(o - C::BV) : C::VOFF + (o - C::BV);
      return kso + (o - C::BS);
    };
    if constexpr (KF16) {
      for (int i = lane; i < 4 * G_; i += 64) {  // fp16 key: 8-dim run (g, j) = (i / 4, i % 4)
        const int off = 1024 * (i >> 2) + 16 * (16 * (i & 3) + tnew);
        *reinterpret_cast<u32x4*>(dst + at(off)) = *reinterpret_cast<const u32x4*>(tokblk + off);
      }
    } else {
      for (int i = lane; i < 4 * G_; i += 64) {  // K index dwords: chunk q = 4g + j
        const int off = (16 * (i & 3) + tnew) * 4 * G_ + 4 * (i >> 2);
        *reinterpret_cast<uint32_t*>(dst + at(off)) = *reinterpret_cast<const uint32_t*>(tokblk + off);
      }
    }
    if (keys_only) {
      if (!KF16 && lane < G_) {  // the token's K scales
        const int off = C::BS + 2 * (tnew * G_ + lane);
        *reinterpret_cast<f16*>(dst + at(off)) = *reinterpret_cast<const f16*>(tokblk + off);
      }
      return;
    }
    if constexpr (VB == 4) {
      for (int c = lane; c < D / 2; c += 64) {  // V index bytes: dim pair c = 16g + m
        const int off = C::BV + (16 * (tnew >> 2) + (c & 15)) * 4 * G_ + 4 * (c >> 4) + (tnew & 3);
        dst[at(off)] = tokblk[off];
      }
    } else {  // packed values: byte tnew % 4 of the X dwords of rows 16j..16j+15 (and of Z)
      constexpr int XD = G_ >= 2 ? G_ / 2 : 1;
      const int j = tnew >> 2, e = tnew & 3;
      for (int i = lane; i < 16 * XD; i += 64) {
        const int off = C::BV + 4 * (16 * j * XD + i) + e;
        dst[at(off)] = tokblk[off];
      }
      if constexpr (VB == 3) {
        for (int i = lane; i < 4 * G_; i += 64) {  // Z dwords (l*G + g)/4 of those rows
          const int off = C::BV + 128 * G_ + 4 * (4 * j * G_ + i) + e;
          dst[at(off)] = tokblk[off];
        }
      }
    }
    constexpr int NSCL = KF16 ? G_ : 2 * G_;  // scales of the token: (K then) V
    if (lane < NSCL) {
      const int off = C::BS + (lane >= G_ ? 32 * G_ : 0) + 2 * (tnew * G_ + (lane % G_));
      *reinterpret_cast<f16*>(dst + at(off)) = *reinterpret_cast<const f16*>(tokblk + off);
    }
  };
  // Pages are issued in order; nis = next page number to issue. The ring fills up over the
  // first steps (at most 4 issues per step) instead of in one burst that would stall the
  // prologue behind a full memory queue.
  int nis = min(npw, 2);
  // Keep the waves abreast on long loops. The hardware lets the oldest waves issue first, so
  // the youngest ones otherwise finish last, alone on their SIMDs and with too few pages in
  // flight. A wave that lags the furthest one (by page-loop step) takes issue priority.
  const bool balance = npw >= 32;
  auto balance_step = [&](int na) {
    int lead = 0;
    if (lane == 0) lead = atomicMax(&lead_n, na);
    const int lag = __builtin_amdgcn_readfirstlane(lead) - na;
    if (lag >= 4) __builtin_amdgcn_s_setprio(3);
    else if (lag >= 2) __builtin_amdgcn_s_setprio(2);
    else __builtin_amdgcn_s_setprio(0);
  };
  // Register path: a page set's scale blocks (PPS per set) go to the wave's first ring slot,
  // where the score and value steps read them: the X set's first, the Y set's after them,
  // or, where both sets' do not fit one slot (sparse, 2-bit values), in the wave's second
  // slot (until a wave writes its results, its slots are its own)
  uint8_t* const ssw = &ring[0][wv][0];
  uint8_t* const ssy = 2 * PPS * C::SCB <= C::SLOT ? ssw + PPS * C::SCB : &ring[1][wv][0];
  auto put_scales = [&](uint8_t* ss, const uint32_t (&sw)[PPS][SW]) {
#pragma unroll
    for (int i = 0; i < PPS; i++)
#pragma unroll
      for (int c = 0; c < SW; c++)
        if (64 * c + lane < C::SCB / 4) reinterpret_cast<uint32_t*>(ss + i * C::SCB)[64 * c + lane] = sw[i][c];
  };
  // Sparse values, register path, first pass: the scores of a step's two pages (keys in
  // registers, K scales in the set's scale blocks), each page's largest score per head
  // into pmreg as kstep does, and the running max and sum.
  auto kstepN = [&](const uint32_t (&kk)[PPS][RG], const uint8_t* ss, int na_, const int (&pg)[PPS]) {
    if constexpr (REG && SPV) {
      static_assert(PPS % 2 == 0, "the page maxima are kept per page pair");
#pragma unroll
      for (int j = 0; j < NPR; j++) {  // pair j: wave pages na_ + 2j (A) and na_ + 2j + 1 (B)
        float sA[4], sB[4], sc[4];
        scores_w(kk[2 * j], ss + 2 * j * C::SCB, 0, sA);
        scores_w(kk[2 * j + 1], ss + (2 * j + 1) * C::SCB, 0, sB);
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const float own = hiLane ? sA[e] : sB[e];
          const float sup = hiLane ? sB[e] : sA[e];
          sc[e] = own + dpp_ror8(sup);
        }
        const int ga = pg[2 * j], gb = pg[2 * j + 1];
        if (ga >= p1 || ga == ptail || gb >= p1 || gb == ptail) {  // wave-uniform
          const int pm = hiLane ? ga : gb;
          const int lim = (pm >= p1) ? 0 : (pm == ptail ? ltail : 16);
#pragma unroll
          for (int e = 0; e < 4; e++)
            if (4 * jq + e >= lim) sc[e] = -INFINITY;
        }
        float pmx = vmax3(sc[0], sc[1], vmax(sc[2], sc[3]));
        pmx = max_xor16(pmx);
        pmx = max_xor32(pmx);  // this lane's page (A if hiLane), head hl: its largest score
        const int na2 = na_ + 2 * j;
        const int kreg = na2 >> 3, kq = (na2 >> 1) & 3;
#pragma unroll
        for (int k = 0; k < NPM; k++)
          pmreg[k] = (k == kreg && jq == kq) ? pmx : pmreg[k];
        const float cm = vmax(pmx, dpp_ror8(pmx));  // both pages
        if (__any(cm > m_run)) {
          const float mn = fmaxf(m_run, cm);
          l_run *= __builtin_amdgcn_exp2f((m_run - mn) * down);  // 2^-inf = 0
          m_run = mn;
          nmd = -mn * down;
        }
#pragma unroll
        for (int e = 0; e < 4; e++) l_run += __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e], down, nmd));
      }
    }
  };
  // The appended token (block layout in tokblk) into the registers of the page that holds
  // it: lane l holds the K index dwords of token l % 16, in byte e of each V index dword
  // the token 4 (l / 16) + e, and scale dword l (and 64 + l) of the block, whose two
  // halves belong to one token.
  auto patch_regs = [&](uint32_t (&k)[RG], uint32_t (&v)[VRG], uint32_t (&sw)[SW]) {
    if constexpr (REG) {  // (register pages only)
      if ((lane & 15) == tnew) {
#pragma unroll
        for (int g = 0; g < RG; g++) k[g] = *reinterpret_cast<const uint32_t*>(tokblk + lane * 4 * G + 4 * g);
      }
      if ((lane >> 4) == (tnew >> 2)) {
        const uint32_t m = 0xFFu << (8 * (tnew & 3));
        if constexpr (VB == 4) {
#pragma unroll
          for (int g = 0; g < RG; g++)
            v[g] = (v[g] & ~m) | (*reinterpret_cast<const uint32_t*>(tokblk + C::BV + lane * 4 * G + 4 * g) & m);
        } else {  // packed: byte tnew % 4 of the lane's X dwords (and of its Z dword)
#pragma unroll
          for (int i = 0; i < XD; i++)
            v[i] = (v[i] & ~m) | (*reinterpret_cast<const uint32_t*>(tokblk + C::BV + 4 * (lane * XD + i)) & m);
          if constexpr (VB == 3) {
            const int zd = G == 2 ? lane >> 1 : lane;
            v[XD] = (v[XD] & ~m) | (*reinterpret_cast<const uint32_t*>(tokblk + C::BV + 128 * G + 4 * zd) & m);
          }
        }
      }
#pragma unroll
      for (int c = 0; c < SW; c++) {
        const int d = 64 * c + lane;                 // scale dword: halves 2d, 2d + 1
        const int hv = 2 * d - (2 * d >= 16 * G ? 16 * G : 0);  // half index inside K or V scales
        if (d < C::SCB / 4 && hv / G == tnew)
          sw[c] = *reinterpret_cast<const uint32_t*>(tokblk + C::BS + 4 * d);
      }
    }
  };
  // The same for sparse values' first pass, whose page registers hold only the K index
  // dwords and K scale dwords l (and 64 + l) of the block (lanes past the K scales hold a
  // copy of the last one)
  auto patch_keys = [&](uint32_t (&k)[RG], uint32_t (&sw)[SW]) {
    if ((lane & 15) == tnew) {
#pragma unroll
      for (int g = 0; g < RG; g++) k[g] = *reinterpret_cast<const uint32_t*>(tokblk + lane * 4 * G + 4 * g);
    }
#pragma unroll
    for (int c = 0; c < SW; c++) {
      const int d = 64 * c + lane;  // K scale dword: halves 2d, 2d + 1 of token 2d / G
      if (d < C::SCB / 8 && (2 * d) / G == tnew)
        sw[c] = *reinterpret_cast<const uint32_t*>(tokblk + C::BS + 4 * d);
    }
  };
  if constexpr (SPV) {
    // Sparse values [mlxcel manual, sparse-V threshold]. Pass 1 streams the keys of every
    // page of this wave (exact running max and sum, page maxima). The workgroup's maximum
    // per head M (over every wave: deterministic) then decides: a page is kept if some
    // live head has 2^((max score - M) * down) >= v_thr; every other token's final weight,
    // exp(s - m_final) / l with m_final >= M and l >= 1, is below v_thr too. Pass 2 streams
    // keys and values of the kept pages through the dense step with the maximum fixed at M,
    // and the sum over every token comes from pass 1. (At most 32 pages per wave: the split
    // count is chosen for it.)
    if constexpr (REG) {
      // keys only, through registers: the X and Y sets alternate as in the dense loop
      auto krun = [&](int st, uint32_t (&k)[PPS][RG], uint32_t (&sw)[PPS][SW], uint8_t* ss) {
        int pg[PPS];
#pragma unroll
        for (int i = 0; i < PPS; i++) pg[i] = p0 + wv + NW * (PPS * st + i);
        if (app && wv == wl) {  // wave-uniform: the appended token's key into its page
          wait_token();
#pragma unroll
          for (int i = 0; i < PPS; i++)
            if (pg[i] == plast) patch_keys(k[i], sw[i]);
        }
        put_scales(ss, sw);
        kstepN(k, ss, PPS * st, pg);
      };
      const int nst = (npw + PPS - 1) / PPS;
      int st = 0;
#pragma unroll 1
      for (; st + 2 < nst; st += 2) {
        krun(st, xk, xs, ssw);
        ldkstep(st + 2, xk, xs);
        krun(st + 1, yk, ys, ssy);
        ldkstep(st + 3, yk, ys);
      }
      if (st < nst) krun(st, xk, xs, ssw);
      if (st + 1 < nst) krun(st + 1, yk, ys, ssy);
    } else {
#pragma unroll 1
      for (int na = 0; na < npw; na += 2) {
        const int nmax = min(npw, na + NR);
#pragma unroll
        for (int k = 0; k < 4; k++)
          if (nis < nmax) {
            stage_keys(nis);
            nis++;
          }
        wait_pages_in_flight<SplitDma<D, KCODEC, VB>::NK_OPS, NR - 2>(max(0, min(NR - 2, nis - na - 2)));
        const int pa = p0 + wv + NW * na;
        if (app && wv == wl && (pa == plast || pa + NW == plast)) {  // wave-uniform
          wait_token();
          copy_token(const_cast<uint8_t*>(k_slot(pa == plast ? na : na + 1)), true, true,
                     C::HS ? C::KREG : C::SOFF);
          asm volatile("" ::: "memory");
        }
        kstep(na, k_slot(na), k_slot(na + 1), pa, pa + NW);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (jq == 0 && hr < 8) mml[wv][hr][0] = m_run;
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; w++) M = fmaxf(M, mml[w][hl][0]);
    // The unit's maximum so far decides which pages are skipped: every split publishes its
    // own per head (an atomic max on an order-preserving integer image, in the workspace's
    // zeroed counter area) and reads the largest published. It is at most the unit's final
    // maximum, so a page below the threshold relative to it is below it relative to the
    // final one too; the last split to arrive clears the entries again.
    if (ns > 1 && wv == 0 && lane < 8) {
      const uint32_t bits = __float_as_uint(M);
      const uint32_t e = (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
      uint32_t* slot = reinterpret_cast<uint32_t*>(a.counters) + TQ_SPARSE_MAX_BASE + 8 * u + lane;
      const uint32_t o = max(e, __hip_atomic_fetch_max(slot, e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      mpub[lane] = __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
    }
    __syncthreads();  // (mml is written again in the epilogue)
    const float Mu = ns > 1 ? mpub[hl] : M;
    const float l_all = (m_run == -INFINITY) ? 0.0f : l_run * __builtin_amdgcn_exp2f((m_run - M) * down);
    m_run = M;
    nmd = -M * down;
    // keep mask: bit n = page n of this wave
    const float l2t = __builtin_amdgcn_logf(a.v_thr);  // log2 of the threshold
    uint32_t keep = 0;
#pragma unroll
    for (int k = 0; k < NPM; k++) {
      const int n = 8 * k + (lane >> 3);
      const bool hit = live && n < npw && (pmreg[k] - Mu) * down >= l2t;
      const uint64_t bal = __ballot(hit);
#pragma unroll
      for (int q = 0; q < 8; q++)
        if ((bal >> (8 * q)) & 0xffu) keep |= 1u << (8 * k + q);
    }
    keep = __builtin_amdgcn_readfirstlane(keep);
    const int nk = __builtin_popcount(keep);
    nskip = npw - nk;
    int klist = 0;  // lane i: the wave page number of the i-th kept page
    {
      uint32_t m = keep;
      for (int i = 0; m != 0u; i++) {
        const int n = __builtin_ctz(m);
        m &= m - 1u;
        if (lane == i) klist = n;
      }
    }
    auto kn = [&](int i) { return __builtin_amdgcn_readlane(klist, i); };
    if constexpr (REG) {
      // the kept pages, PPS at a time, keys and values into the X set (few: one wait each)
#pragma unroll 1
      for (int i = 0; i < nk; i += PPS) {
        int pg[PPS];
#pragma unroll
        for (int j = 0; j < PPS; j++) {
          const bool kept = i + j < nk;
          const int n = kept ? kn(i + j) : npw;  // past the end: a dummy load, masked below
          ldp(n, xk[j], xv[j], xs[j]);
          pg[j] = kept ? p0 + wv + NW * n : p1;
        }
        if (app && wv == wl) {  // wave-uniform: the appended token into its page, if kept
          wait_token();
#pragma unroll
          for (int j = 0; j < PPS; j++)
            if (pg[j] == plast) patch_regs(xk[j], xv[j], xs[j]);
        }
        put_scales(ssw, xs);
        stepN(xk, xv, ssw, pg);
      }
    } else {
      int nis2 = 0;
#pragma unroll 1
      for (int i = 0; i < nk; i += 2) {
        const int nmax = min(nk, i + NSLOT);
#pragma unroll
        for (int k = 0; k < 4; k++)
          if (nis2 < nmax) {
            stage_page<D, KCODEC, VB>(page_blk(kn(nis2)), slot_lds(nis2 % NSLOT), lane);
            nis2++;
          }
        wait_pages_in_flight<C::NDMA, NSLOT - 2>(max(0, min(NSLOT - 2, nis2 - i - 2)));
        const int pa = p0 + wv + NW * kn(i);
        const int pb = (i + 1 < nk) ? p0 + wv + NW * kn(i + 1) : p1;  // p1: no page B
        if (app && wv == wl && (pa == plast || pb == plast)) {  // wave-uniform
          wait_token();
          copy_token(ring[(pa == plast ? i : i + 1) % NSLOT][wv], true);
          asm volatile("" ::: "memory");
        }
        step(ring[i % NSLOT][wv], ring[(i + 1) % NSLOT][wv], pa, pb);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    l_run = l_all;
    if (lane == 0 && nskip > 0) atomicAdd(&wskip, nskip);  // (one global add per workgroup below)
  } else if constexpr (REG) {
    // Register path: step st over the X set, step st + 1 over the Y set; each set is
    // reloaded (two steps ahead) as soon as its step is done.
    // One step over a set. The last step of a wave is the only one that can hold the
    // sequence's last page (pages ascend), so only it carries the fused append's patch.
    auto run_step = [&](auto last, int st, uint32_t (&k)[PPS][RG], uint32_t (&v)[PPS][VRG],
                        uint32_t (&sw)[PPS][SW], uint8_t* ss) {
      if (balance) balance_step(PPS * st);
      const int pa0 = p0 + wv + NW * PPS * st;
      if constexpr (decltype(last)::value) {
        if (app && wv == wl) {  // wave-uniform
          wait_token();
#pragma unroll
          for (int i = 0; i < PPS; i++)
            if (pa0 + NW * i == plast) patch_regs(k[i], v[i], sw[i]);
        }
      }
      put_scales(ss, sw);
      int pg[PPS];
#pragma unroll
      for (int i = 0; i < PPS; i++) pg[i] = pa0 + NW * i;
      stepN(k, v, ss, pg);
    };
    const int nst = (npw + PPS - 1) / PPS;  // steps of this wave
    // The loop runs the steps that are not the last; the last one or two run after it.
    int st = 0;
#pragma unroll 1
    for (; st + 2 < nst; st += 2) {
      run_step(std::false_type{}, st, xk, xv, xs, ssw);
      ldstep(st + 2, xk, xv, xs);
      run_step(std::false_type{}, st + 1, yk, yv, ys, ssy);
      ldstep(st + 3, yk, yv, ys);
    }
    if (st + 1 < nst) {
      run_step(std::false_type{}, st, xk, xv, xs, ssw);
      run_step(std::true_type{}, st + 1, yk, yv, ys, ssy);
    } else if (st < nst) {
      run_step(std::true_type{}, st, xk, xv, xs, ssw);
    }
  } else {
#pragma unroll 1
  for (int na = 0; na < npw; na += 2) {
    if (balance) balance_step(na);
    const int nmax = min(npw, na + NSLOT);  // the slots of pages < na are free again
#pragma unroll
    for (int k = 0; k < 4; k++)
      if (nis < nmax) {
        stage_page<D, KCODEC, VB>(page_blk(nis), slot_lds(nis % NSLOT), lane);
        nis++;
      }
    const int younger = max(0, min(NSLOT - 2, nis - na - 2));  // pages issued after page na + 1
    wait_pages_in_flight<C::NDMA, NSLOT - 2>(younger);
    const int pa = p0 + wv + NW * na;
    if (app && wv == wl && (pa == plast || pa + NW == plast)) {  // wave-uniform
      wait_token();
      copy_token(ring[(pa == plast ? na : na + 1) % NSLOT][wv], true);
      asm volatile("" ::: "memory");
    }
    step(ring[na % NSLOT][wv], ring[(na + 1) % NSLOT][wv], pa, pa + NW);
  }
  }

  __builtin_amdgcn_s_setprio(0);
  if (app && wv == wc)  // the appended token goes to the pool too, for later calls
    copy_token(const_cast<uint8_t*>(a.pool) + ((int64_t)__builtin_amdgcn_readfirstlane(pid_last) * a.Hkv + h) * BB, false);

  // ---- epilogue: merge the waves of this workgroup -----------------------------------------
  l_run = sum_xor16(l_run);
  l_run = sum_xor32(l_run);
  l_run += dpp_ror8(l_run);  // lanes hr and hr ^ 8 summed the two pages of each step
  m_run *= down;  // to the log2 domain of the merges below
  // back from the subnormal operand units: even dims carry 2^-24, odd dims 2^-20
#pragma unroll
  for (int g = 0; g < G; g++) {
    acc[2 * g] *= 16777216.0f;
    acc[2 * g + 1] *= 1048576.0f;
  }
  // This wave's page loop is over, so its ring slots are free: its results go there now,
  // while the other waves may still be streaming pages through theirs.
  if (hr < 8) {
#pragma unroll
    for (int g = 0; g < G; g++) {
      // dims 32g + 8jq + 0..7: even dims from acc[2g], odd from acc[2g+1]
      float* dst = mo(wv, hr) + 32 * g + 8 * jq;
      const f32x4 lo4 = {acc[2 * g][0], acc[2 * g + 1][0], acc[2 * g][1], acc[2 * g + 1][1]};
      const f32x4 hi4 = {acc[2 * g][2], acc[2 * g + 1][2], acc[2 * g][3], acc[2 * g + 1][3]};
      *reinterpret_cast<f32x4*>(dst) = lo4;
      *reinterpret_cast<f32x4*>(dst + 4) = hi4;
    }
    if (jq == 0) {
      mml[wv][hr][0] = m_run;
      mml[wv][hr][1] = l_run;
    }
  }
  __syncthreads();  // every wave's results are in
  if (SPV && tid == 0 && a.v_skipped && wskip > 0) atomicAdd(a.v_skipped, (unsigned long long)wskip);
  if (tid < 128) {  // per head, one row of 16 lanes (lane = wave): weights 2^(m_w - M)
    const int hd = tid >> 4, w = tid & 15;   // into mml[w][hd][0], and the sum l
    const bool on = hd < r && w < NW;
    const float mw = on ? mml[w][hd][0] : -INFINITY;
    float M = mw;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) M = fmaxf(M, lane_xor16(M, o, lane));
    const float f = (mw == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
    float l = on ? f * mml[w][hd][1] : 0.0f;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) l += lane_xor16(l, o, lane);
    if (on) mml[w][hd][0] = f;
    if (on && w == 0) {
      hml[hd][0] = M;
      hml[hd][1] = l;
    }
  }
  __syncthreads();
  int nwsum = NW;  // waves whose results are summed below
  if (!SPV && tsl > 0) {
    // This split's slice of the fp16 tail [mlxcel manual, delegated cache]: scores with the
    // query as given, p = 2^(s - M_t) in the log2 domain as the pages' scores, values summed
    // in the original basis and rotated into the cache basis (sign flip, butterflies, rho),
    // then joined to the pages' result of this workgroup by the usual max/rescale rule.
    float* qs = reinterpret_cast<float*>(&ring[0][0][0] + MEND + 8 * TQ_MAX_SPLITS * 4);
    float* ps = qs + 8 * D;           // [8][TQ_MAX_HOT] scores, then weights
    float* pw = ps + 8 * TQ_MAX_HOT;  // [8][D] the pages' part: sum over waves of f_w o_w
    const int64_t qh = ((int64_t)b * a.Hq + (int64_t)h * r) * D;
    const f16* hk = static_cast<const f16*>(a.hot_k) + (((int64_t)b * a.Hkv + h) * a.hot_cap + t0) * D;
    const f16* hv = static_cast<const f16*>(a.hot_v) + (((int64_t)b * a.Hkv + h) * a.hot_cap + t0) * D;
    const float qmul2 = a.attn_scale * TQ_LOG2E;
    // Scores: 8 lanes per token, lane sg holding dims [sg D/8, (sg+1) D/8) (KP loads of 8),
    // wave wv taking tokens tb + (lane / 8), tb = 8 wv, 8 wv + 8 NW, ...
    // Values: a lane holds 4 consecutive dims (chunk c) of one of TPW consecutive tokens (j);
    // wave wv takes the token rows wv, wv + NW, ... of TPW tokens each, HB of them per batch.
    // The first keys and values are loaded before anything else, so that their latency
    // overlaps the folding of the pages' result.
    constexpr int KP = D / 64, CH = D / 4, TPW = 64 / CH > 1 ? 64 / CH : 1, HB = 8;
    const int tt = lane >> 3, sg = lane & 7;
    const int c = lane % CH, j = lane / CH;
    f16x8 kp[KP];
    f16x4 v4[HB];
    auto load_k = [&](int tb) {
      const int t = tb + tt;
      if (t < tsl) {
#pragma unroll
        for (int i = 0; i < KP; i++)
          kp[i] = *reinterpret_cast<const f16x8*>(hk + (int64_t)t * D + sg * (D / 8) + 8 * i);
      }
    };
    auto load_v = [&](int n0) {
#pragma unroll
      for (int k = 0; k < HB; k++) {
        const int t = (n0 + k * NW) * TPW + j;
        if (t < tsl) v4[k] = *reinterpret_cast<const f16x4*>(hv + (int64_t)t * D + 4 * c);
      }
    };
    // (the query first: the loads complete in order, so its wait would cover the others)
    constexpr int QPT = (8 * D + NT - 1) / NT;
    float qx[QPT];
#pragma unroll
    for (int k = 0; k < QPT; k++) {
      const int i = tid + k * NT;
      qx[k] = (i < 8 * D && i < r * D) ? load_q(a.q, a.q_dtype, qh + i) * qmul2 : 0.0f;
    }
    load_k(8 * wv);
    load_v(wv);
#pragma unroll
    for (int k = 0; k < QPT; k++) {
      const int i = tid + k * NT;
      if (i < 8 * D) {
        const int hd = i / D, d = i - hd * D;
        float o = 0.0f;
        if (hd < r) {
#pragma unroll
          for (int w = 0; w < NW; w++) o += mml[w][hd][0] * mo(w, hd)[d];
        }
        pw[i] = o;
        qs[i] = qx[k];
      }
    }
    __syncthreads();
    for (int tb = 8 * wv; tb < tsl; tb += 8 * NW) {
      f16x8 kc[KP];  // this pass's keys; the next pass's are loaded meanwhile
#pragma unroll
      for (int i = 0; i < KP; i++) kc[i] = kp[i];
      if (tb + 8 * NW < tsl) load_k(tb + 8 * NW);
      float dot[8] = {};
#pragma unroll
      for (int i = 0; i < KP; i++)
#pragma unroll
        for (int e = 0; e < 8; e++) {
          const float kx = (float)kc[i][e];
          const int d = sg * (D / 8) + 8 * i + e;
#pragma unroll
          for (int hd = 0; hd < 8; hd++) dot[hd] = __builtin_fmaf(qs[hd * D + d], kx, dot[hd]);
        }
#pragma unroll
      for (int hd = 0; hd < 8; hd++) {
        dot[hd] += lane_xor16(dot[hd], 1, lane);
        dot[hd] += lane_xor16(dot[hd], 2, lane);
        dot[hd] += lane_xor16(dot[hd], 4, lane);
      }
      const int t = tb + tt;
      if (t < tsl && sg < r) {
        float v = dot[0];
#pragma unroll
        for (int hd = 1; hd < 8; hd++) v = sg == hd ? dot[hd] : v;
        ps[sg * TQ_MAX_HOT + t] = v;
      }
    }
    __syncthreads();
    float Mt = -INFINITY, lt = 0.0f;  // wave hd: the slice's max and sum for head hd
    if (wv < r) {
      float* pr = ps + wv * TQ_MAX_HOT;
      for (int t = lane; t < tsl; t += 64) Mt = fmaxf(Mt, pr[t]);
      Mt = wave_max(Mt);
      for (int t = lane; t < tsl; t += 64) {
        const float p = __builtin_amdgcn_exp2f(pr[t] - Mt);
        pr[t] = p;
        lt += p;
      }
      lt = wave_sum(lt);
    }
    __syncthreads();
    {
      float acc[8][4] = {};
      const int nrow = (tsl + TPW - 1) / TPW;
      for (int n0 = wv; n0 < nrow; n0 += NW * HB) {
        f16x4 vc[HB];  // this batch's values; the next batch's are loaded meanwhile
#pragma unroll
        for (int k = 0; k < HB; k++) vc[k] = v4[k];
        if (n0 + NW * HB < nrow) load_v(n0 + NW * HB);
#pragma unroll
        for (int k = 0; k < HB; k++) {
          const int t = (n0 + k * NW) * TPW + j;
          if (t < tsl) {
#pragma unroll
            for (int hd = 0; hd < 8; hd++) {
              const float p = hd < r ? ps[hd * TQ_MAX_HOT + t] : 0.0f;
#pragma unroll
              for (int e = 0; e < 4; e++) acc[hd][e] = __builtin_fmaf(p, (float)vc[k][e], acc[hd][e]);
            }
          }
        }
      }
      // the TPW token lanes of each chunk, then the waves (through mo, whose page results
      // are folded into pw above)
#pragma unroll
      for (int m = CH; m < 64; m <<= 1)
#pragma unroll
        for (int hd = 0; hd < 8; hd++)
#pragma unroll
          for (int e = 0; e < 4; e++) acc[hd][e] += xor_shfl(acc[hd][e], m);
      if (j == 0) {
#pragma unroll
        for (int hd = 0; hd < 8; hd++)
          if (hd < r) *reinterpret_cast<f32x4*>(mo(wv, hd) + 4 * c) = f32x4{acc[hd][0], acc[hd][1], acc[hd][2], acc[hd][3]};
      }
    }
    __syncthreads();
    if (wv < r) {  // wave hd: the slice into the cache basis, joined to the pages' part
      float x[V];
#pragma unroll
      for (int k = 0; k < V; k++) {
        const int d = lane + 64 * k;
        float o = 0.0f;
        for (int w = 0; w < NW; w++) o += mo(w, wv)[d];
        x[k] = ((sgn_s[d >> 5] >> (d & 31)) & 1u) ? -o : o;
      }
      wave_fwht<V>(x, lane);
      const float Mp = hml[wv][0], lp = hml[wv][1];
      const float M = fmaxf(Mp, Mt);
      const float cp = (Mp == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(Mp - M);
      const float ct = __builtin_amdgcn_exp2f(Mt - M);
#pragma unroll
      for (int k = 0; k < V; k++) {
        const int d = lane + 64 * k;
        mo(0, wv)[d] = cp * pw[wv * D + d] + ct * (x[k] * rho);
      }
      if (lane == 0) {
        hml[wv][0] = M;
        hml[wv][1] = cp * lp + ct * lt;
        mml[0][wv][0] = 1.0f;
      }
    }
    nwsum = 1;
    __syncthreads();
  }
  // fin: [ngf][r][D] partial sums of the result (rotated basis), summed by the rotation below
  float* fin = reinterpret_cast<float*>(&ring[0][0][0]);
  int ngf = 1;
  const int S = a.splits + a.hot_wg;  // partial rows per unit
  const int64_t prow = ((int64_t)u * S + srow) * r;  // partial rows of this (unit, split)
  if (ns == 1) {
    float ov[(8 * D + NT - 1) / NT];
#pragma unroll
    for (int j = 0; j < (8 * D + NT - 1) / NT; j++) {
      const int i = tid + j * NT;
      float o = 0.0f;
      if (i < r * D) {
        const int hd = i / D, d = i % D;
#pragma unroll
        for (int w = 0; w < NW; w++)
          if (w < nwsum) o += mml[w][hd][0] * mo(w, hd)[d];
        o /= hml[hd][1];
      }
      ov[j] = o;
    }
    __syncthreads();  // fin aliases mo
#pragma unroll
    for (int j = 0; j < (8 * D + NT - 1) / NT; j++)
      if (tid + j * NT < r * D) fin[tid + j * NT] = ov[j];
  } else {
    for (int i = tid; i < r * D; i += NT) {
      const int hd = i / D, d = i % D;
      float o = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; w++)
        if (w < nwsum) o += mml[w][hd][0] * mo(w, hd)[d];
      __hip_atomic_store(&a.part_o[(prow + hd) * D + d], o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (d == 0) {
        __hip_atomic_store(&a.part_ml[2 * (prow + hd)], hml[hd][0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&a.part_ml[2 * (prow + hd) + 1], hml[hd][1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    // Publish this split without a cache write-back: the partials were stored coherently at
    // device scope (sc1), vmcnt(0) waits for them, then the arrival counter is bumped.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0)
      last_flag = (__hip_atomic_fetch_add(&a.counters[u], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == ns - 1);
    __syncthreads();
    if (!last_flag) return;
    if (tid == 0) __hip_atomic_store(&a.counters[u], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (SPV && tid < 8)  // every split of the unit has read the published maxima
      __hip_atomic_store(reinterpret_cast<uint32_t*>(a.counters) + TQ_SPARSE_MAX_BASE + 8 * u + tid, 0u,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // ---- the last workgroup of unit u merges every split (coherent sc1 loads) ----------
    // thread = (split group grp, head hd, 4 dims d4); split group grp takes splits
    // grp, grp + ngrp, ...; the first NLD of them are loaded before the weights are known.
    // Wave hd (< r) first loads the (m, l) of every split of head hd (lanes over splits), so
    // that they arrive ahead of the partials and the weights 2^(m_t - M) / sum_t 2^(m_t - M) l_t
    // are computed while the partials are still loading.
    const int64_t row0 = (int64_t)u * S * r;
    __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(a.part_o + row0 * D, (short)0, S * r * D * 4, 0x00020000);
    constexpr int D4 = D / 4;
    const int ngrp = max(1, NT / (r * D4));
    ngf = ngrp;
    const bool act = tid < ngrp * r * D4;
    const int grp = tid / (r * D4), hd = (tid / D4) % r, d4 = tid % D4;
    constexpr int TPL = TQ_MAX_SPLITS / 64;  // splits per lane
    float m[TPL], l[TPL];
    if (wv < r) {
#pragma unroll
      for (int q = 0; q < TPL; q++) {
        const int t = lane + 64 * q;
        m[q] = -INFINITY;
        l[q] = 0.0f;
        if (t < ns) {
          m[q] = __hip_atomic_load(&a.part_ml[2 * (row0 + (int64_t)t * r + wv)], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          l[q] = __hip_atomic_load(&a.part_ml[2 * (row0 + (int64_t)t * r + wv) + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    // Partials of split t, or zero for t >= ns and inactive threads: an offset past the
    // descriptor's range reads nothing and returns zeros. The loads stay unconditional, so
    // that waiting for the (m, l) loads above does not wait for them too.
    constexpr int NLD = 16;  // split loads in flight per thread
    auto load_part = [&](int t) {
      const uint32_t off = (act && t < ns) ? (uint32_t)(((t * r + hd) * D + 4 * d4) * 4) : 0x80000000u;
      return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, off, 0, 16));
    };
    f32x4 v[NLD];
#pragma unroll
    for (int k = 0; k < NLD; k++) v[k] = load_part(grp + k * ngrp);
    if (wv < r) {
      float M = m[0];
#pragma unroll
      for (int q = 1; q < TPL; q++) M = fmaxf(M, m[q]);
      M = wave_max(M);
      float lsum = 0.0f;
#pragma unroll
      for (int q = 0; q < TPL; q++) {
        m[q] = (m[q] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m[q] - M);
        lsum += m[q] * l[q];
      }
      const float inv = 1.0f / wave_sum(lsum);
#pragma unroll
      for (int q = 0; q < TPL; q++)
        if (lane + 64 * q < ns) wsh[wv][lane + 64 * q] = m[q] * inv;
    }
    __syncthreads();
    f32x4 o4 = {0.0f, 0.0f, 0.0f, 0.0f};
    if (act) {
#pragma unroll
      for (int k = 0; k < NLD; k++)
        if (grp + k * ngrp < ns) o4 += wsh[hd][grp + k * ngrp] * v[k];
      for (int t0 = grp + NLD * ngrp; t0 < ns; t0 += NLD * ngrp) {  // more splits per group
#pragma unroll
        for (int k = 0; k < NLD; k++) v[k] = load_part(t0 + k * ngrp);
#pragma unroll
        for (int k = 0; k < NLD; k++)
          if (t0 + k * ngrp < ns) o4 += wsh[hd][t0 + k * ngrp] * v[k];
      }
    }
    __syncthreads();  // fin aliases mo
    if (act) *reinterpret_cast<f32x4*>(&fin[(grp * r + hd) * D + 4 * d4]) = o4;
  }
  __syncthreads();
  // ---- back to the original basis: wave w takes head w (fp32 butterflies, rho, sigma) -------
  if (wv < r) {
    float x[V];
#pragma unroll
    for (int k = 0; k < V; k++) {
      float o = 0.0f;
      for (int g2 = 0; g2 < ngf; g2++) o += fin[(g2 * r + wv) * D + lane + 64 * k];
      x[k] = o;
    }
    wave_fwht<V>(x, lane);
#pragma unroll
    for (int k = 0; k < V; k++) {
      const int d = lane + 64 * k;
      const float y = x[k] * rho;
      outp[wv * D + d] = ((sgn_s[d >> 5] >> (d & 31)) & 1u) ? -y : y;
    }
  }
}

// n int32 zeros from p (a plain fill kernel: usable where a memset node is not wanted).
__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t* __restrict__ p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0;
}

// Longest-first order of the units (b, h), for grids larger than the chip holds at once,
// where a long sequence whose workgroups start last would finish alone: position p takes
// head p % Hkv of the sequence ranked p / Hkv by context length (longest first, ties by
// index). Positions keep the XCD placement of the decode grid.
__global__ __launch_bounds__(256) void lpt_order_kernel(const int32_t* __restrict__ lens, int B,
                                                        int Hkv, int32_t* __restrict__ order) {
  __shared__ int lens_s[TQ_LPT_MAX_BATCH];
  __shared__ int seq_of_rank[TQ_LPT_MAX_BATCH];
  const int t = threadIdx.x;
  if (t < B) lens_s[t] = lens[t];
  __syncthreads();
  if (t < B) {
    const int lt = lens_s[t];
    int rank = 0;
    for (int j = 0; j < B; j++) {
      const int lj = lens_s[j];
      rank += (lj > lt || (lj == lt && j < t)) ? 1 : 0;
    }
    seq_of_rank[rank] = t;
  }
  __syncthreads();
  for (int p = t; p < B * Hkv; p += 256) order[p] = seq_of_rank[p / Hkv] * Hkv + p % Hkv;
}

template <int D, int VB, bool SPV>
hipError_t launch_dqs(const LaunchDecode& a, hipStream_t st, unsigned grid) {
  constexpr int VC = VB == 4 ? TQ_CODEC_ABSMAX : (VB == 3 ? TQ_CODEC_ABSMAX3 : TQ_CODEC_ABSMAX2);
  if (a.k_codec == TQ_CODEC_FP16) {
    // fp16 keys: 8 waves, 4 at D = 256 (three staged pages per wave must fit the LDS ring)
    constexpr int NWF = tq_decode_waves(D, TQ_CODEC_FP16, VC, SPV);
    hipLaunchKernelGGL((decode_fused<D, TQ_CODEC_FP16, VB, NWF, SPV>), dim3(grid), dim3(64 * NWF), 0, st, a);
  } else if (a.k_codec == TQ_CODEC_LLOYDMAX) {
    constexpr int NW = tq_decode_waves(D, TQ_CODEC_LLOYDMAX, VC, SPV);
    hipLaunchKernelGGL((decode_fused<D, TQ_CODEC_LLOYDMAX, VB, NW, SPV>), dim3(grid), dim3(64 * NW), 0, st, a);
  } else {
    constexpr int NW = tq_decode_waves(D, TQ_CODEC_ABSMAX, VC, SPV);
    hipLaunchKernelGGL((decode_fused<D, TQ_CODEC_ABSMAX, VB, NW, SPV>), dim3(grid), dim3(64 * NW), 0, st, a);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const LaunchDecode& a, hipStream_t st) {
  if (a.order) {
    if (a.B > TQ_LPT_MAX_BATCH) return hipErrorInvalidValue;
    hipLaunchKernelGGL(lpt_order_kernel, dim3(1), dim3(256), 0, st, a.context_lens, a.B, a.Hkv, a.order);
  }
  const int U = a.B * a.Hkv;
  const unsigned grid = (unsigned)(8 * ((U + 7) / 8) * (a.splits + a.hot_wg));
  const int vb = tq_value_bits(a.v_codec);
  if (a.sparse_v) {
    if (vb == 3) return launch_dqs<D, 3, true>(a, st, grid);
    if (vb == 2) return launch_dqs<D, 2, true>(a, st, grid);
    return launch_dqs<D, 4, true>(a, st, grid);
  }
  if (vb == 3) return launch_dqs<D, 3, false>(a, st, grid);
  if (vb == 2) return launch_dqs<D, 2, false>(a, st, grid);
  return launch_dqs<D, 4, false>(a, st, grid);
}

}  // namespace

hipError_t tq_launch_zero_i32(int32_t* p, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int blocks = std::min((n + 255) / 256, 1024);
  hipLaunchKernelGGL(zero_i32_kernel, dim3(blocks), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

hipError_t tq_launch_decode(const LaunchDecode& a, hipStream_t st) {
  switch (a.D) {
    case 64: return launch_d<64>(a, st);
    case 128: return launch_d<128>(a, st);
    default: return launch_d<256>(a, st);
  }
}
