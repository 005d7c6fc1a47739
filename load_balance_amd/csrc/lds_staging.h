// Device helpers shared by the attention kernels for gfx950: row tiles staged in LDS by
// direct global -> LDS copies and read back as MFMA operands, in both orientations.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace lb {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Raw buffer resource word 3 for gfx9-family dword loads (no format conversion).
constexpr int kBufferFlags = 0x00020000;

// Row tiles (keys, values or query rows) are copied from global memory straight into LDS by
// the buffer loads' LDS mode: no registers, no stores, several stages in flight in a ring.
// A tile is stored row-major and unpadded, each row's 16-byte chunks XOR-permuted by the row
// (swz), and serves both MFMA operand shapes: row fragments (8 consecutive d of one row) for
// the products that contract over d, and transposed fragments (one d column of 8 rows) for
// those that contract over the rows, read with gfx950's LDS transpose load
// (ds_read_b64_tr_b16: each lane receives one column of 4 rows, the 16 lanes of a group
// supplying the 4 x 16 block's row addresses).
//
// The chunk permutation of row r (r mod 16 decides it).  Row reads: 16 lanes read one
// logical chunk of 16 consecutive rows, which land on 16 distinct chunk slots (d = 128) or on
// 8 slots in each bank half (d = 64: two rows per 256 bytes).  Transpose reads: 32 lanes read
// four logical chunks (a 64-byte run) of 4 consecutive rows, which land on 4 disjoint runs.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }  // s_waitcnt vmcnt(n) only

// Raw buffer resource over [base, base + nbytes): reads past the end return zeros.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, int nbytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)p),
               __builtin_amdgcn_readfirstlane((int)((p >> 32) & 0xFFFF)), __builtin_amdgcn_readfirstlane(nbytes),
               kBufferFlags};
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (int)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p));
}

// Copies global -> LDS without registers: lane i's 16 (or 4) bytes at voffset land at
// lds + 16 i (or 4 i).  Written as inline assembly on purpose: the compiler, seeing the
// builtin's LDS write, would wait for every copy in flight before each LDS read of the loop;
// the kernel waits for its copies itself (vmcnt) before the barrier that publishes a stage.
// The copy takes its LDS address from m0, which the statement restores.  `lds` must be
// wave-uniform (it is read from the first active lane, so that the compiler can keep it in
// a scalar register wherever it cannot prove it uniform).
__device__ __forceinline__ void copy16_to_lds(i32x4 rsrc, uint32_t lds, int voffset) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voffset), "s"(rsrc)
      : "memory");
}
__device__ __forceinline__ void copy4_to_lds(i32x4 rsrc, uint32_t lds, int voffset) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dword %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voffset), "s"(rsrc)
      : "memory");
}

// Row fragment: 8 consecutive d (logical chunk `chunk`) of row `row` of a swizzled tile.
template <int D>
__device__ __forceinline__ bf16x8 row_frag(const char* tile, int row, int chunk) {
  return *reinterpret_cast<const bf16x8*>(tile + row * (D * 2) + ((chunk ^ swz<D>(row)) << 4));
}

// Transposed fragment (the A operand of an MFMA contracting over rows): for the lane's
// column d = 32 db + lane % 32, rows r0 + 8 t' + 4 hh + j (t' = 0, 1; j = 0..3) as elements
// 4 t' + j, hh = lane / 32.  Each half is one transpose load: in a group of 16 lanes, lane i
// supplies row r0 + 8 t' + 4 hh + i / 4 at columns 32 db + 16 (group % 2) + 4 (i % 4).
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const char* tile, int r0, int db, int lane) {
  const int lg = lane & 15, gq = (lane >> 4) & 1, hh = lane >> 5;
  const int col = db * 32 + 16 * gq + 4 * (lg & 3);
  bf16x4 h[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int row = r0 + 8 * q + 4 * hh + (lg >> 2);
    const char* p = tile + row * (D * 2) + (((col >> 3) ^ swz<D>(row)) << 4) + (col & 7) * 2;
    h[q] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
  }
  return __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7);
}

// The same fragments with the lane's address arithmetic done once: for a fragment whose first
// row r0 is a multiple of 16, rows r0 + i land on the chunk permutation of row i (swz reads
// r mod 16 only), so each fragment is a lane offset fixed for the tile, per 32-wide d block
// and half, plus r0 * 2D bytes, which the LDS read takes as its immediate offset.
template <int D>
struct TrOffsets {
  int off[D / 32][2];
  __device__ __forceinline__ void init(int lane) {
    const int lg = lane & 15, gq = (lane >> 4) & 1, hh = lane >> 5;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int col = db * 32 + 16 * gq + 4 * (lg & 3);
        const int row = 8 * q + 4 * hh + (lg >> 2);
        off[db][q] = row * (D * 2) + (((col >> 3) ^ swz<D>(row)) << 4) + (col & 7) * 2;
      }
  }
};
// tr_frag(tile, r0, db, lane) for r0 a multiple of 16
template <int D>
__device__ __forceinline__ bf16x8 tr_frag_at(const char* tile, const TrOffsets<D>& o, int r0, int db) {
  bf16x4 h[2];
#pragma unroll
  for (int q = 0; q < 2; ++q)
    h[q] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(tile + o.off[db][q] + r0 * (D * 2)));
  return __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7);
}

// One wave's share of copying a tile of ROWS rows of one head of a [row][heads][D] bf16 tensor
// (row_step bytes per row) into LDS: the tile's 1 KB pieces are spread evenly over 8 waves,
// and every wave issues the same count, kCopies.  The lane offsets are computed once; a copy
// then costs the tile's base address, one buffer resource and the copy instructions.  Rows
// from `valid` on read as zeros (the buffer range ends there).
template <int D, int ROWS>
struct TileCopier {
  static constexpr int kChunks = D / 8, kRowsPerCopy = 1024 / (D * 2);
  static constexpr int kCopies = ROWS * D * 2 / 1024 / 8;
  static_assert(ROWS * D * 2 % (1024 * 8) == 0, "the pieces must divide evenly over 8 waves");
  int voff[kCopies];  // the lane's byte offset in the source, from the tile's first row of its head
  uint32_t loff;      // the wave's first piece in the tile (wave-uniform)

  __device__ __forceinline__ void init(int64_t row_step, int wave, int lane) {
    wave = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
    for (int j = 0; j < kCopies; ++j) {
      const int row = (wave * kCopies + j) * kRowsPerCopy + lane / kChunks;
      const int chunk = (lane % kChunks) ^ swz<D>(row);  // lane writes slot lane % kChunks of its row
      voff[j] = row * (int)row_step + chunk * 16;
    }
    loff = __builtin_amdgcn_readfirstlane(wave * kCopies * 1024);
  }
  // rows [r0, r0 + ROWS) of head `head` into the tile at LDS address `lds`
  __device__ __forceinline__ void issue(const void* src, int64_t row_step, int r0, int valid, int head,
                                        uint32_t lds) const {
    const char* base = reinterpret_cast<const char*>(src) + (int64_t)r0 * row_step + (int64_t)head * D * 2;
    const i32x4 rs = buffer_rsrc(base, valid * (int)row_step);
#pragma unroll
    for (int j = 0; j < kCopies; ++j) copy16_to_lds(rs, lds + loff + j * 1024, voff[j]);
  }
  // the same copy with the lane offsets computed on the spot, for kernels that cannot spare
  // the registers that keep them
  __device__ __forceinline__ static void issue_now(const void* src, int64_t row_step, int r0, int valid, int head,
                                                   uint32_t lds, int wave, int lane) {
    TileCopier c;
    c.init(row_step, wave, lane);
    c.issue(src, row_step, r0, valid, head, lds);
  }
};

// s_waitcnt vmcnt(k * per) for k = min(2, younger) stages still allowed in flight
__device__ __forceinline__ void wait_stage(int younger, int per) {
  if (younger >= 2) {
    if (per == 5) __builtin_amdgcn_s_waitcnt(vmcnt_imm(10));
    else if (per == 4) __builtin_amdgcn_s_waitcnt(vmcnt_imm(8));
    else if (per == 3) __builtin_amdgcn_s_waitcnt(vmcnt_imm(6));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(4));
  } else if (younger == 1) {
    if (per == 5) __builtin_amdgcn_s_waitcnt(vmcnt_imm(5));
    else if (per == 4) __builtin_amdgcn_s_waitcnt(vmcnt_imm(4));
    else if (per == 3) __builtin_amdgcn_s_waitcnt(vmcnt_imm(3));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(2));
  } else {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }
}

}  // namespace
}  // namespace lb
