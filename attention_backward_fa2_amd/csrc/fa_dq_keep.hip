// fa_dq_keep.hip -- the instantiations of the dQ kernel of fa_dq.hip that
// read the forward's dropout keep words, in a translation unit of their own
// so that they compile in parallel with the rest.
#define FA_TU_DROPOUT 2
#include "fa_dq.hip"
