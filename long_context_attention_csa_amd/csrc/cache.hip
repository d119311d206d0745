// State-cache maintenance for resuming a sequence at a prefix (cf-1.com
// write-up §4.4: the KV cache is split into a state cache and a classical KV
// cache, with three trade-offs for the recent uncompressed tokens: full SWA
// caching, periodic checkpointing every 1024 tokens, and zero SWA caching).
//
// The state cache of a sequence is the set of rings its decode steps keep:
// the window ring (recent raw KV rows, csa_window_append) and the compressor
// state rings (csa_compress_append, hca_compress_append). The classical cache
// (compressed entries) is complete for every finished block and needs no
// strategy. The kernels here move a sequence's ring contents:
//   checkpoint  after the token at position p is appended, sequences with
//               (p + 1) % period == 0 copy their ring into checkpoint slot
//               (p + 1) / period - 1 (periodic checkpointing);
//   restore     a sequence's ring from a chosen checkpoint slot;
//   ring_fill   a ring rebuilt from a full-length history of its rows (full
//               SWA caching keeps every token's rows).
// Zero SWA caching needs no kernel: the state is rebuilt by appending the
// recent tokens again (appends are bit-identical to the first time).
// All three are plain 16-byte copies driven by device-side positions, so a
// decode step that includes them can be captured in a HIP graph.
#include "common.hpp"

namespace csa {

// One block per (sequence, 4096-byte piece); 256 threads x 16 bytes.
constexpr int kCopyPiece = 4096;

__global__ __launch_bounds__(256) void k_state_checkpoint(const uint8_t* __restrict__ state, int64_t seq_bytes,
                                                          const int32_t* __restrict__ pos, int period,
                                                          uint8_t* __restrict__ ckpt, int64_t n_slots) {
  const int64_t b = blockIdx.y;
  const int64_t p = pos[b];
  if (p < 0 || (p + 1) % period != 0) return;
  const int64_t slot = (p + 1) / period - 1;
  if (slot >= n_slots) return;
  const int64_t off = (int64_t)blockIdx.x * kCopyPiece + 16 * threadIdx.x;
  if (off >= seq_bytes) return;
  *reinterpret_cast<i32x4*>(ckpt + (b * n_slots + slot) * seq_bytes + off) =
      *reinterpret_cast<const i32x4*>(state + b * seq_bytes + off);
}

__global__ __launch_bounds__(256) void k_state_restore(const uint8_t* __restrict__ ckpt, int64_t seq_bytes,
                                                       int64_t n_slots, const int32_t* __restrict__ slot,
                                                       uint8_t* __restrict__ state) {
  const int64_t b = blockIdx.y;
  const int64_t s = slot[b];
  if (s < 0 || s >= n_slots) return;
  const int64_t off = (int64_t)blockIdx.x * kCopyPiece + 16 * threadIdx.x;
  if (off >= seq_bytes) return;
  *reinterpret_cast<i32x4*>(state + b * seq_bytes + off) =
      *reinterpret_cast<const i32x4*>(ckpt + (b * n_slots + s) * seq_bytes + off);
}

// ring[b, t mod R] = hist[b, t] for t in [max(0, pos[b] - R), pos[b]), rows
// of row_bytes; one block per (sequence, ring row), 16 bytes per thread.
__global__ __launch_bounds__(256) void k_ring_fill(const uint8_t* __restrict__ hist, int64_t T_hist,
                                                   int64_t row_bytes, const int32_t* __restrict__ pos, int64_t R,
                                                   uint8_t* __restrict__ ring) {
  const int64_t b = blockIdx.y, i = blockIdx.x;   // i-th of the last R positions before pos
  const int64_t p = pos[b];
  const int64_t t = p - R + i;
  if (p < 0 || t < 0 || t >= p || t >= T_hist) return;
  const uint8_t* src = hist + (b * T_hist + t) * row_bytes;
  uint8_t* dst = ring + (b * R + t % R) * row_bytes;
  for (int64_t off = 16 * (int64_t)threadIdx.x; off < row_bytes; off += 16 * 256)
    *reinterpret_cast<i32x4*>(dst + off) = *reinterpret_cast<const i32x4*>(src + off);
}

hipError_t launch_state_checkpoint(const void* state, int64_t B, int64_t seq_bytes, const int32_t* pos, int period,
                                   void* ckpt, int64_t n_slots, hipStream_t s) {
  const dim3 grid((unsigned)cdiv(seq_bytes, kCopyPiece), (unsigned)B);
  k_state_checkpoint<<<grid, 256, 0, s>>>(static_cast<const uint8_t*>(state), seq_bytes, pos, period,
                                          static_cast<uint8_t*>(ckpt), n_slots);
  return hipGetLastError();
}

hipError_t launch_state_restore(const void* ckpt, int64_t B, int64_t seq_bytes, int64_t n_slots, const int32_t* slot,
                                void* state, hipStream_t s) {
  const dim3 grid((unsigned)cdiv(seq_bytes, kCopyPiece), (unsigned)B);
  k_state_restore<<<grid, 256, 0, s>>>(static_cast<const uint8_t*>(ckpt), seq_bytes, n_slots, slot,
                                       static_cast<uint8_t*>(state));
  return hipGetLastError();
}

hipError_t launch_ring_fill(const void* hist, int64_t B, int64_t T_hist, int64_t row_bytes, const int32_t* pos,
                            int64_t R, void* ring, hipStream_t s) {
  const dim3 grid((unsigned)R, (unsigned)B);
  k_ring_fill<<<grid, 256, 0, s>>>(static_cast<const uint8_t*>(hist), T_hist, row_bytes, pos, R,
                                   static_cast<uint8_t*>(ring));
  return hipGetLastError();
}

}  // namespace csa
