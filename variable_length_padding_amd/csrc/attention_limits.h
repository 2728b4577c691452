// Addressing limit of the head_dim 64/128 attention kernel (attention.hip),
// in a plain C++ header so that the host can test it without a GPU.
#pragma once

#include <cstdint>

namespace ee {

constexpr int kAttnKeyTile = 32;  // keys per LDS tile of the attention kernels

// attn_tr_kernel addresses a sequence's key and value rows with signed 32-bit
// byte offsets from the sequence's first row: row k0 + r of a key tile (k0 a
// multiple of the tile below the sequence length L, r < kAttnKeyTile), times
// the row stride in bytes, plus a 16-byte chunk of the row's head slice.  The
// largest is below (max_len - 1 + kAttnKeyTile) * row_stride * 2 + row_stride
// * 2; the kernel runs only when that fits, else the 64-bit addressed kernel
// does.  Rows past L fall outside the buffer descriptor's range and read 0.
inline bool attn_tr_offsets_fit(int64_t max_len, int64_t row_stride_halves) {
  return (max_len + kAttnKeyTile) * row_stride_halves * 2 < (int64_t(1) << 31);
}

}  // namespace ee
