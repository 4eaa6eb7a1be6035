// LDS tiles of K/V rows for the gfx950 kernels: direct global->LDS loads
// (global_load_lds_dwordx4, no staging registers) into a multi-stage ring,
// and the MFMA operand reads out of it.
//
// One tile = 64 consecutive (or gathered) K/V rows of d bf16 values.
//   K tile: row-major, 16-byte unit u of row r stored at unit u ^ (r mod units
//           per row), which spreads the MFMA operand reads (32 rows, same
//           unit) over all LDS banks.
//   V tile: d-block major, [d/32][64 rows][32 values]: the transpose reads of a
//           16-lane group then touch 4 rows x 32 bytes in distinct banks, and
//           every read of a lane is one base address plus an immediate offset.
// A direct LDS load writes lane i's 16 bytes at (wave-uniform base + 16 i), so
// a layout is produced by choosing which global 16 bytes each lane loads.
#pragma once

#include "mage_common.hpp"

namespace mage {

template <int D, int kNT = kThreads>
struct TileGeom {
  static constexpr int kRowBytes = D * 2;                         // K row
  static constexpr int kUnits = D / 8;                            // 16-byte units per K row
  static constexpr int kBytes = kTileKeys * kRowBytes;            // one K (or V) tile
  static constexpr int kInstr = kBytes / (kNT * 16);              // DMA instructions per wave
  static constexpr int kVBlock = kTileKeys * 64;                  // one 32-value d block of V
  static_assert(kInstr >= 1, "tile smaller than one DMA round");
};

// s_waitcnt with only vmcnt limited to N (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

// Work-group barrier without the memory fence that __syncthreads() implies
// (that fence would wait for every outstanding LDS DMA load); the asm memory
// clobbers keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Hand-off between the work-groups of one launch through a counter. What is
// handed over is stored and read only with agent-scope cache bits (sc1): the
// instructions the compiler emits for relaxed agent-scope atomic stores and
// loads, which its gfx942/gfx950 memory model makes coherent across the XCDs'
// L2s by the scope bits alone. Its agent-scope release adds a write-back of
// the XCD's L2 (buffer_wbl2) before the wait for completion, for plain stores
// that may sit dirty there; with no plain stores to publish, the wait alone
// orders the handed-over stores before the count: every thread's stores
// drain (vmcnt 0: performed at agent scope), the work-group meets, one lane
// counts in. The work-group that brings the count to n (zeroing the counter
// when `reset`) gets true in every thread and reads the data with sc1 loads,
// issued after the count's result returned. With the compiler's release and
// acquire fences instead, the later step takes 1.2 us longer at 128K context.
__device__ __forceinline__ bool count_in(uint32_t* counter, uint32_t n, bool reset, int32_t* s_flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t before = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = before == n - 1;
    if (last && reset) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = last;
  }
  __syncthreads();
  return *s_flag != 0;
}

// Wait until at most `pending` tiles (of kPerTile DMA instructions each) are
// still in flight for this wave; pending <= kStages - 1.
template <int kPerTile, int P>
__device__ __forceinline__ void wait_tiles_impl(int pending) {
  if constexpr (P == 0) {
    wait_vmcnt<0>();
  } else {
    if (pending >= P)
      wait_vmcnt<kPerTile * P>();
    else
      wait_tiles_impl<kPerTile, P - 1>(pending);
  }
}

template <int kPerTile, int kStages>
__device__ __forceinline__ void wait_tiles(int pending) {
  static_assert(kPerTile * (kStages - 1) < 64, "vmcnt is 6 bits");
  wait_tiles_impl<kPerTile, kStages - 1>(pending);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)(p)));
}

// Direct LDS loads with a wave-uniform 64-bit base (SGPR pair) and a per-lane
// 32-bit byte offset: lane i's 16 bytes at base + off_i land at LDS address
// lds + 16 i. Written as one asm block so that the VGPR offsets stay the
// loop-invariant registers the caller keeps them in, and M0 (the LDS base
// register of the instruction) is set inside the block; the s_nop covers the
// wait state between an M0 write and its use. Completion is tracked with
// vmcnt by the caller (wait_vmcnt / wait_tiles). Nothing is returned in a
// register, so nothing is live while the loads are in flight.
// kNt1: the second load is non-temporal (cache policy nt: its lines are
// streamed, not kept, so they do not evict data that is read again soon).
template <bool kNt1 = false>
__device__ __forceinline__ void dma16x2(const void* b0, uint32_t o0, uint32_t l0, const void* b1, uint32_t o1,
                                        uint32_t l1) {
  l0 = __builtin_amdgcn_readfirstlane(l0);   // wave-uniform; kept in SGPRs for M0
  l1 = __builtin_amdgcn_readfirstlane(l1);
  if constexpr (kNt1) {
    asm volatile(
        "s_mov_b32 m0, %4\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1\n\t"
        "s_mov_b32 m0, %5\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %3 nt"
        :
        : "v"(o0), "s"(b0), "v"(o1), "s"(b1), "s"(l0), "s"(l1)
        : "memory", "m0");
  } else {
    asm volatile(
        "s_mov_b32 m0, %4\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1\n\t"
        "s_mov_b32 m0, %5\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %3"
        :
        : "v"(o0), "s"(b0), "v"(o1), "s"(b1), "s"(l0), "s"(l1)
        : "memory", "m0");
  }
}

// A single load of the dma16x2 form (kNt: non-temporal).
template <bool kNt = false>
__device__ __forceinline__ void dma16(const void* b, uint32_t o, uint32_t l) {
  l = __builtin_amdgcn_readfirstlane(l);
  if constexpr (kNt) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1 nt"
        :
        : "v"(o), "s"(b), "s"(l)
        : "memory", "m0");
  } else {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(o), "s"(b), "s"(l)
        : "memory", "m0");
  }
}

// One direct LDS load per lane from a per-lane 64-bit address, waited for in
// the same asm block (the path for tiles whose rows are not contiguous in
// memory; the wait frees the address registers before the block ends).
template <bool kNt = false>
__device__ __forceinline__ void dma16_sync(const void* addr, uint32_t lds) {
  lds = __builtin_amdgcn_readfirstlane(lds);
  if constexpr (kNt) {
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off nt\n\t"
        "s_waitcnt vmcnt(0)"
        :
        : "v"(addr), "s"(lds)
        : "memory", "m0");
  } else {
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off\n\t"
        "s_waitcnt vmcnt(0)"
        :
        : "v"(addr), "s"(lds)
        : "memory", "m0");
  }
}

// Issue the DMA loads of one tile. row_off(r) returns the element offset of
// tile row r (0..63) in the K/V arrays; it must always name a readable row.
template <int D, bool kWithV, int kNT = kThreads, class RowOff>
__device__ __forceinline__ void issue_tile(uint8_t* k_lds, uint8_t* v_lds, const uint16_t* kbase,
                                           const uint16_t* vbase, RowOff row_off, int w, int lane) {
  using G = TileGeom<D, kNT>;
#pragma unroll
  for (int j = 0; j < G::kInstr; ++j) {
    const int slot = w * G::kInstr + j;                // 1 KiB slice of the tile
    const int unit = slot * kWave + lane;              // 16-byte unit index in the tile
    {
      const int r = unit / G::kUnits, phys = unit % G::kUnits;
      const int uk = phys ^ (r & (G::kUnits - 1));
      __builtin_amdgcn_global_load_lds(kbase + row_off(r) + uk * 8, k_lds + slot * 1024, 16, 0, 0);
    }
    if constexpr (kWithV) {
      // slot -> d block slot/4, rows 16*(slot%4) + lane/4, 16-byte unit lane%4
      const int db = slot >> 2, r = ((slot & 3) << 4) + (lane >> 2);
      __builtin_amdgcn_global_load_lds(vbase + row_off(r) + 32 * db + 8 * (lane & 3),
                                       v_lds + slot * 1024, 16, 0, 0);
    }
  }
}

// Per-lane byte offsets (inside a K tile) of the MFMA operand fragments of
// row `row`: ofs[ks] holds d values 16*ks + 8*hh .. +7.
template <int D>
__device__ __forceinline__ void k_frag_offsets(int row, int hh, uint32_t (&ofs)[D / 16]) {
  using G = TileGeom<D>;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    ofs[ks] = row * G::kRowBytes + (((2 * ks + hh) ^ (row & (G::kUnits - 1))) << 4);
}

// K fragments at tile base `base` + ofs[ks] + kImm. The reads and their wait
// sit in one asm block: as builtins, the compiler would also wait for every
// outstanding direct-to-LDS load before them and drain the load ring.
template <int D, int kImm>
__device__ __forceinline__ void k_frags(uint32_t base, const uint32_t (&ofs)[D / 16],
                                        bf16x8 (&f)[D / 16]) {
  uint32_t a[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) a[ks] = base + ofs[ks];
  u32x4 r[D / 16];
  if constexpr (D == 128) {
    asm volatile(
        "ds_read_b128 %0, %8 offset:%16\n\t"
        "ds_read_b128 %1, %9 offset:%16\n\t"
        "ds_read_b128 %2, %10 offset:%16\n\t"
        "ds_read_b128 %3, %11 offset:%16\n\t"
        "ds_read_b128 %4, %12 offset:%16\n\t"
        "ds_read_b128 %5, %13 offset:%16\n\t"
        "ds_read_b128 %6, %14 offset:%16\n\t"
        "ds_read_b128 %7, %15 offset:%16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
          "=&v"(r[6]), "=&v"(r[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]),
          "i"(kImm));
  } else {
    static_assert(D == 64, "head_dim 64 or 128");
    asm volatile(
        "ds_read_b128 %0, %4 offset:%8\n\t"
        "ds_read_b128 %1, %5 offset:%8\n\t"
        "ds_read_b128 %2, %6 offset:%8\n\t"
        "ds_read_b128 %3, %7 offset:%8\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(kImm));
  }
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) f[ks] = __builtin_bit_cast(bf16x8, r[ks]);
}

// LDS pointer of a byte address (LDS pointers are 32-bit).
template <class T>
__device__ __forceinline__ __attribute__((address_space(3))) T* lds_ptr(uint32_t addr) {
  return (__attribute__((address_space(3))) T*)(addr);
}

// k_frags as ordinary LDS loads, for loops whose tile loads are all asm DMA:
// the compiler then tracks these reads itself, issues them early and waits
// (lgkmcnt) only where a fragment is first used.
template <int D>
__device__ __forceinline__ void k_frags_lds(uint32_t base, const uint32_t (&ofs)[D / 16], bf16x8 (&f)[D / 16]) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) f[ks] = __builtin_bit_cast(bf16x8, *lds_ptr<const u32x4>(base + ofs[ks]));
}

// Per-lane byte offset of the V^T fragment reads (inside a V tile). Each
// fragment takes two ds_read_b64_tr_b16: within each 16-lane group the
// hardware hands lane i element i%4 of the 8 bytes loaded by lanes i/4 + 4j,
// so lane l ends up with 8 keys of one d column (the A operand of
// v_mfma_f32_32x32x16_bf16 for V^T).
__device__ __forceinline__ uint32_t vt_lane_offset(int lane) {
  const int q = lane >> 4, sg = lane & 15;
  return ((8 * (q >> 1) + (sg >> 2)) << 6) + ((q & 1) << 5) + ((sg & 3) << 3);
}

// All V^T fragments of one 32-key half tile: frag[db][s] holds in lane l the
// values V[32h + 16s + 8*(l/32) + j][32*db + (l%32)], j = 0..7 (vaddr includes
// the half's offset and the lane's transpose-read offset). One asm block, one
// wait, 4 * D/32 transpose reads. kB is the byte stride of one 32-value d
// block: 64 rows x 64 bytes in a 64-key tile, 32 x 64 in a 32-key tile.
template <int D, int kB = kTileKeys * 64>
__device__ __forceinline__ void vt_frags_half(uint32_t vaddr, bf16x8 (&frag)[D / 32][2]) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  typedef short s8 __attribute__((ext_vector_type(8)));
  if constexpr (D == 128) {
    s4 r[16];
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16 offset:0\n\t"
        "ds_read_b64_tr_b16 %1, %16 offset:256\n\t"
        "ds_read_b64_tr_b16 %2, %16 offset:1024\n\t"
        "ds_read_b64_tr_b16 %3, %16 offset:1280\n\t"
        "ds_read_b64_tr_b16 %4, %16 offset:%17\n\t"
        "ds_read_b64_tr_b16 %5, %16 offset:%18\n\t"
        "ds_read_b64_tr_b16 %6, %16 offset:%19\n\t"
        "ds_read_b64_tr_b16 %7, %16 offset:%20\n\t"
        "ds_read_b64_tr_b16 %8, %16 offset:%21\n\t"
        "ds_read_b64_tr_b16 %9, %16 offset:%22\n\t"
        "ds_read_b64_tr_b16 %10, %16 offset:%23\n\t"
        "ds_read_b64_tr_b16 %11, %16 offset:%24\n\t"
        "ds_read_b64_tr_b16 %12, %16 offset:%25\n\t"
        "ds_read_b64_tr_b16 %13, %16 offset:%26\n\t"
        "ds_read_b64_tr_b16 %14, %16 offset:%27\n\t"
        "ds_read_b64_tr_b16 %15, %16 offset:%28\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
          "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]),
          "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15])
        : "v"(vaddr), "i"(kB), "i"(kB + 256), "i"(kB + 1024), "i"(kB + 1280), "i"(2 * kB),
          "i"(2 * kB + 256), "i"(2 * kB + 1024), "i"(2 * kB + 1280), "i"(3 * kB),
          "i"(3 * kB + 256), "i"(3 * kB + 1024), "i"(3 * kB + 1280));
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const s4 lo = r[4 * db + 2 * s2], hi = r[4 * db + 2 * s2 + 1];
        frag[db][s2] = __builtin_bit_cast(bf16x8, s8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      }
  } else {
    static_assert(D == 64, "head_dim 64 or 128");
    s4 r[8];
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:0\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:256\n\t"
        "ds_read_b64_tr_b16 %2, %8 offset:1024\n\t"
        "ds_read_b64_tr_b16 %3, %8 offset:1280\n\t"
        "ds_read_b64_tr_b16 %4, %8 offset:%9\n\t"
        "ds_read_b64_tr_b16 %5, %8 offset:%10\n\t"
        "ds_read_b64_tr_b16 %6, %8 offset:%11\n\t"
        "ds_read_b64_tr_b16 %7, %8 offset:%12\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
          "=&v"(r[6]), "=&v"(r[7])
        : "v"(vaddr), "i"(kB), "i"(kB + 256), "i"(kB + 1024), "i"(kB + 1280));
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const s4 lo = r[4 * db + 2 * s2], hi = r[4 * db + 2 * s2 + 1];
        frag[db][s2] = __builtin_bit_cast(bf16x8, s8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      }
  }
}

// vt_frags_half as compiler-visible transpose loads (same fragments and
// addresses), for the same loops as k_frags_lds.
template <int D, int kB = kTileKeys * 64>
__device__ __forceinline__ void vt_frags_half_lds(uint32_t vaddr, bf16x8 (&frag)[D / 32][2]) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  typedef short s8 __attribute__((ext_vector_type(8)));
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const uint32_t a = vaddr + db * kB + s2 * 1024;
      const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr<s4>(a));
      const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr<s4>(a + 256));
      frag[db][s2] = __builtin_bit_cast(bf16x8, s8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    }
}

}  // namespace mage
