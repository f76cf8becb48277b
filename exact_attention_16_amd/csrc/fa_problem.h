// What one launch of the attention-forward kernels computes, as plain data:
// pointers, element strides, optional per-sequence offsets and sizes. Plain
// C++ (no HIP): the kernels take it by value, and the host-side validation
// fills and checks it (that code also builds with an ordinary C++ compiler).
#pragma once

namespace fa {

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;

// Strides are in elements; a row is D contiguous elements. Without
// per-sequence offsets (cuq == nullptr) sequence b, head h has Sq query rows
// starting at q + b*qb + h*qh (row stride qs) and Sk key rows in k and v
// likewise; o has q's row count and lse is Sq floats at lse + b*lb + h*lh.
// With offsets, sequence b's query rows are token rows cuq[b] .. cuq[b+1]-1
// (so its rows start at q + cuq[b]*qs + h*qh, lse + h*lh + cuq[b]) and its
// key rows are token rows cuk[b] .. cuk[b+1]-1; the kernel clamps both ranges
// to the totq / totk token rows the tensors hold and the lengths to Sq / Sk.
struct Problem {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  long long qb, qh, qs, kb, kh, ks, vb, vh, vs, ob, oh, os, lb, lh;
  const int* cuq;
  const int* cuk;
  int totq, totk;
  int B, H, Sq, Sk;
  int nqt;  // query tiles per (sequence, head) for the kernel's block of rows
  float c;  // scale * log2(e) (8-bit inputs: times the Q and K descales)
  unsigned long long* events;  // rescale-event counter of the diagnostic kernels
  float vscale;  // 8-bit inputs: the V descale, applied to O at the end
  int hgroup;    // causal: heads an XCD takes together (block_to_tile)
  int items;     // work items (Q tile, sequence, head) the launch runs
  int compact;   // variable lengths: items are only the query tiles within
                 // each sequence (varlen_tile in fa_layout.h), else all
                 // nqt * B * H of them
};

}  // namespace fa
