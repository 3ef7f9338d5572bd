// Page-table loader: one block-table read per page, one 64-bit page base.
//
// A sequence's keys live in pages of `page_size` tokens; slot s of its
// block-table row names the physical page that holds tokens
// [s * page_size, (s + 1) * page_size).  The loader follows the per-page
// design of rocm-libraries "one K/V resource per page on the gfx942 2D i64
// path" (Technical Details, Changes): the page id is read once for the whole
// page and every copy from that page is (page base, offset inside the page).
// Differences from that design, for gfx950:
//  * the id is read by the wave with a uniform (scalar) load and is never
//    re-read per copy, so no wait on it drains the in-flight K/V loads;
//  * the base is the zero-extended id times the page's byte size, formed in
//    64-bit arithmetic, so a cache of any size up to 2^63 bytes is addressed
//    correctly (the page above shows sign extension failing past 2^31 bytes);
//  * only ids of slots below the sequence's own page count ever select a
//    page, a stricter bound than one over the whole table, so an unmapped id
//    in a slot past the sequence (or in the table's tail) is never
//    dereferenced (id_early below reads a slot ahead of that check, inside
//    the row's W slots, and its caller drops the value unless the slot is
//    mapped).
// In-page offsets stay 32-bit: a page is far below 4 GiB.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

struct PageTable {
  const int32_t* row;   // this sequence's block-table row
  int64_t page_bytes;   // bytes of one page of one cache tensor
  int n_pages;          // ceil(seq_len / page_size): slots that may be read

  // Physical page id in slot `slot`, wave-uniform.  The caller guarantees
  // 0 <= slot < n_pages; `slot` is wave-uniform.  The read goes through the
  // constant address space (the table does not change while a kernel runs),
  // which makes it a scalar load even in kernels whose LDS-DMA copies keep
  // the compiler from proving that on its own.
  __device__ __forceinline__ uint32_t id(int slot) const {
    typedef __attribute__((address_space(4))) const int32_t* const_ptr;
    return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(((const_ptr)row)[slot]));
  }
  // Physical page id in slot `slot` read before the sequence's page count is
  // known, so that the read does not wait for the sequence length.  The
  // read stays inside the row's `width` slots (a table with no slots reads
  // `fallback`, any valid int32); its value may be anything unless the
  // caller later finds slot < n_pages, which alone makes it a page id.  For
  // a read at a kernel's start, before anything it issues may write memory:
  // an ordinary load, which the compiler makes a scalar one there and, unlike
  // a read of constant memory, does not repeat where the value is used.
  __device__ __forceinline__ uint32_t id_early(int slot, int width, const int32_t* fallback) const {
    const int32_t* src = width > 0 ? row + (slot < width ? slot : width - 1) : fallback;
    return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(*src));
  }
  // Byte offset of page `page_id` from the start of the cache.
  __device__ __forceinline__ int64_t base_of(uint32_t page_id) const {
    return static_cast<int64_t>(static_cast<uint64_t>(page_id)) * page_bytes;
  }
  // Byte offset of the page in slot `slot` from the start of the cache.
  __device__ __forceinline__ int64_t base(int slot) const { return base_of(id(slot)); }
};

}  // namespace pa
