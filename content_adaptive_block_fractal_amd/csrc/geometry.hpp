// Layer geometry shared by the host-side launchers and the kernels.
//
// The token grid (T frames x H x W) is padded to Hp = Ty*P, Wp = Tx*P and
// reordered patch by patch (NABLA summary, Methodology item 1); each P x P
// patch of a frame is one block of P*P = 64 tokens.
#pragma once

#include <cstdint>

namespace cabf {

constexpr int kP = 8;            // patch side supported by the kernels
constexpr int kBlock = kP * kP;  // tokens per block
constexpr int kMaxBlocks = 8192; // longest block row the mask kernels keep in registers

struct Geo {
  int B, heads, D;      // batch, heads, head_dim
  int T, H, W;          // real grid
  int Ty, Tx;           // patches per column / row of a frame
  int nb;               // blocks per (batch, head)
  int64_t BH;           // batch * heads
  int64_t Nv;           // real tokens per (batch, head): T*H*W
  int64_t N;            // reordered tokens per (batch, head): nb*64
};

}  // namespace cabf
